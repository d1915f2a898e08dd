// Kernels for n_fft = 512: complex FFT of 256 = 16 x 16 points.
#include "fm_backward.h"

namespace fm {
template void* kernel_for<16, 16>(int, int, bool, bool, bool);
template void* backward_kernel_for<16, 16>(int);
}  // namespace fm
