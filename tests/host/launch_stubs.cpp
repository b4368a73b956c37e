// Host-only stand-ins for the kernel launchers of libmla.so, so that the library's host side
// (argument checks, split planner, parameter set-up) can be built and run under the address
// and undefined-behaviour sanitizers on a machine without a GPU.  A call that passes every
// check reaches one of these and gets hipErrorNotSupported back, which the entry point
// reports as MLA_ERR_HIP.
#include "internal.h"
#include "mla.h"

namespace mla {

hipError_t launch_quantize(const float*, uint8_t*, int64_t, float, hipStream_t) {
  return hipErrorNotSupported;
}
int64_t dynamic_quantize_workspace_bytes() { return MLA_QUANTIZE_DYNAMIC_WORKSPACE_BYTES; }
hipError_t launch_quantize_dynamic(const void*, bool, uint8_t*, int64_t, float*, void*,
                                   hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_kv_append(const void*, bool, uint8_t*, int64_t, const int32_t*,
                            const int32_t*, int, int, int, int, float, const float*, const float*,
                            int64_t, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_decode(const DecodeParams& p, int, hipStream_t) {
  // every field the launch would read is read here, so that the sanitizers see them
  volatile int64_t sink = p.batch + p.q_tokens + p.heads + p.rows + p.page_size +
                          p.max_pages + p.num_splits + p.groups + p.page_bytes + p.tiles_hint;
  (void)sink;
  return hipErrorNotSupported;
}
hipError_t launch_read_probe(const void*, int64_t, uint32_t*, int, hipStream_t) {
  return hipErrorNotSupported;
}
int64_t read_probe_chunk_bytes() { return 32768; }
hipError_t launch_combine(const uint16_t*, const float*, int, int, int, float, const float*,
                          uint16_t*, float*, int64_t, bool, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace mla
