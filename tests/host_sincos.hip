// Host build of the library's rotary sin/cos (csrc/common.h), for a CPU test
// that compares them with the C library's long-double sinl/cosl.  Compiled by
// tests/test_host_sincos.py with hipcc for the host only; no GPU code runs.
#include "../cross_context_kv_amd/csrc/common.h"

extern "C" void host_rope_sincos(const double* x, int n, double* s, double* c, float* sf,
                                 float* cf) {
  for (int i = 0; i < n; ++i) {
    kvfix::rope_sincos(x[i], &s[i], &c[i]);
    kvfix::rope_sincos_f32(x[i], &sf[i], &cf[i]);
  }
}
