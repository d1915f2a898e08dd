// Kernels for n_fft = 400: complex FFT of 200 = 8 x 25 points.
#include "fm_backward.h"
#include "fm_rows.h"

namespace fm {
template void* kernel_for<8, 25>(int, int, bool);
template void* backward_kernel_for<8, 25>(int);
template void* rows_kernel_for<25>(int, int);
}  // namespace fm
