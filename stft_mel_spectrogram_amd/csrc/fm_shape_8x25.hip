// Kernels for n_fft = 400: complex FFT of 200 = 8 x 25 points.
#include "fm_backward.h"

namespace fm {
template void* kernel_for<8, 25>(int, int, bool, bool, bool);
template void* backward_kernel_for<8, 25>(int);
}  // namespace fm
