// C ABI of the 3D (HyenaND) path.
#include "../../include/hyena.h"

extern "C" {

size_t hyena_nd_cache_bytes(int, int, int, int, int) { return 0; }
size_t hyena_nd_filter_workspace_bytes(int, int, int, int, int) { return 0; }
size_t hyena_nd_workspace_bytes(int, int, int, int, int, int) { return 0; }
int hyena_nd_layer_init(hyena_nd_layer*, int, int, int, int, int, void*, size_t) { return HYENA_ERR_UNSUPPORTED; }
int hyena_nd_filter_gen(hyena_nd_layer*, const hyena_nd_filter_params*, float*, void*, size_t, hipStream_t) {
  return HYENA_ERR_UNSUPPORTED;
}
int hyena_nd_fwd(const hyena_nd_layer*, const float*, const float*, const float*, const float*, const float*,
                 const float*, int, float*, void*, size_t, hipStream_t) {
  return HYENA_ERR_UNSUPPORTED;
}

}  // extern "C"
