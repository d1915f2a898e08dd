// Kernels for n_fft = 64: complex FFT of 32 = 8 x 4 points.
#include "fm_backward.h"

namespace fm {
template void* kernel_for<8, 4>(int, int, bool, bool, bool);
template void* backward_kernel_for<8, 4>(int);
}  // namespace fm
