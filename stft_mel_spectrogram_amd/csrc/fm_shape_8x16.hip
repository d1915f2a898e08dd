// Kernels for n_fft = 256: complex FFT of 128 = 8 x 16 points.
#include "fm_backward.h"

namespace fm {
template void* kernel_for<8, 16>(int, int, bool, bool, bool);
template void* backward_kernel_for<8, 16>(int);
}  // namespace fm
