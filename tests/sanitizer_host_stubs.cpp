// Launchers for the host-only sanitizer build of libdca (tests/
// test_host_sanitizers.py): the library's host code (api.cpp: validation,
// workspace layout, stage sequencing) is compiled with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer and linked with these
// launchers instead of the HIP kernels. Each reports "no device", the error
// the real launchers return on a machine without a GPU, so every argument
// check runs exactly as in the real library and a valid call ends in
// DCA_E_DEVICE.
#include "dca_internal.h"

namespace dca {

static int no_device() { return (int)hipErrorNoDevice; }

int launch_rope_table(const Problem &, double, void *, const Layout &, void *) { return no_device(); }
int launch_remap(const Problem &, const void *, const void *, const void *, float, void *, const Layout &, void *) {
    return no_device();
}
int launch_vs_index(const Problem &, const dca_vs_mask &, void *, const Layout &, void *) { return no_device(); }
int launch_attention(const Problem &, void *, float *, const void *, const Layout &, void *, const void *) {
    return no_device();
}
int launch_decode(const Problem &, const void *, const void *, const void *, void *, float *, double, float, void *,
                  const Layout &, void *, void *) {
    return no_device();
}
int decode_static_scratch(void *, void **) { return no_device(); }
int launch_vs_estimate(const Problem &, int, int, int, int, const void *, const void *, const Layout &, size_t,
                       float *, float *, int32_t *, int32_t *, void *) {
    return no_device();
}
int launch_debug_positions(int64_t, int64_t, int64_t, int32_t *, int32_t *, int32_t *, int32_t *, void *) {
    return no_device();
}
int launch_debug_tile_regions(int64_t, int64_t, uint8_t *, void *) { return no_device(); }
int launch_debug_unpack(const Problem &, const void *, const Layout &, int, void *, void *) { return no_device(); }
int launch_debug_vs_lists(const Problem &, const void *, const Layout &, int32_t *, int32_t *, int32_t *, int32_t *,
                          void *) {
    return no_device();
}
int launch_debug_vs_tiles(const Problem &, const void *, const Layout &, int, int64_t, int, int32_t *, uint32_t *,
                          int32_t, int32_t *, void *) {
    return no_device();
}

}  // namespace dca
