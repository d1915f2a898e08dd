// Kernels for n_fft = 128: complex FFT of 64 = 8 x 8 points.
#include "fm_backward.h"

namespace fm {
template void* kernel_for<8, 8>(int, int, bool, bool, bool);
template void* backward_kernel_for<8, 8>(int);
}  // namespace fm
