// Large-FFT forward kernel, n_fft/2 = 16 x 16 x 8 (n_fft 4096, beside the
// two-pass kernel of that size; chosen per call).
#include "fm_large.h"

namespace fm {
template void* large_kernel_for<16, 16, 8>(int, int, bool);
}  // namespace fm
