// Launcher of the IQ1_S-like -> IQ1_M-like repacking kernel (k_repack.hip).
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace moe {

hipError_t launch_repack_iq1s(const uint8_t *ql, const uint16_t *qh, const uint16_t *d, size_t n_blocks,
                              uint8_t *ql_out, uint8_t *qh_out, uint64_t *sd_out, hipStream_t s);

}  // namespace moe
