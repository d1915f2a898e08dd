// Large-FFT forward kernel, n_fft/2 = 16 x 16 x 16 (n_fft 8192).
#include "fm_large.h"

namespace fm {
template void* large_kernel_for<16, 16, 16>(int, int, bool);
}  // namespace fm
