// Kernels for n_fft = 1024: complex FFT of 512 = 32 x 16 points.
#include "fm_backward.h"

namespace fm {
template void* kernel_for<32, 16>(int, int, bool, bool, bool);
template void* backward_kernel_for<32, 16>(int);
}  // namespace fm
