// placeholder: replaced by the chunk kernel
#include "kda_common.hpp"
#include "kda_launch.hpp"
namespace kda {
bool chunk_fwd_supported(int, int, int, bool) { return false; }
hipError_t launch_chunk_fwd(const ChunkArgs&) { return hipErrorInvalidValue; }
}
