// Fused mel-spectrogram forward kernel for the largest FFT sizes (n_fft 8192
// and 16384) on gfx950: device code.  fm_large_<a>x<c>x<d>.hip instantiates
// it per shape; fm_launch.hip launches it.
//
// The flashmel 0.1.0 page allows n_fft up to 16384 (README "Usage",
// constraints) and measures a "huge" case at 16384/4096 with 256 mels
// (README "Performance"); it calls these sizes occupancy-bound for a block
// FFT held on chip ("Where each case actually sits").  A frame's complex
// exchange buffer of n_fft/2 points is 32 or 64 KB here, too large for the
// two-register-pass kernel of the smaller sizes (whose second pass keeps two
// whole rows per thread), so the transform runs in three register passes
// over one LDS buffer, one frame at a time per workgroup:
//
// Real FFT of N = n_fft points through the complex FFT of M = N/2 points of
// z[m] = x[2m] + i x[2m+1] (window pre-scaled by 1/2), M = A*C*D, B = C*D:
//   pass 1, thread per b < B:  A-point DFT over a of z[B a + b], times
//           W_M^(b ka), stored at (ka, c, d) with b = D c + d;
//   pass 2, item (ka, d):      C-point DFT over c, times W_B^(d kc),
//           stored at (ka, kc, d);
//   pass 3, item (ka, kc):     D-point DFT over d, stored at (ka, kc, kd),
//           which holds Z[ka + A kc + A C kd];
// then per bin k the real split X[k] = (Z[k] + conj Z[M-k])
// - i W_N^k (Z[k] - conj Z[M-k]) and |X|^p into a power row (aliasing the
// buffer), and the mel projection of that row, thread t taking filters t,
// t + NT, ... over their CSR runs of nonzero weights (copied into LDS behind
// the buffer once per workgroup).  Each pass writes back the positions it
// read, so one buffer serves all three; its strides (D + 1 per c, an odd
// C (D + 1) + 1 per a) put the threads of a pass, and the split's reads of
// consecutive bins, on distinct banks or at most two to a bank.
#pragma once

#include <type_traits>

#include "fm_kernel.h"

namespace fm {

// Kernel arguments (one struct, passed by value).
struct LArgs {
  const void* in;
  void* out;             // [B, n_mels, n_frames] float or _Float16
  const float2* win2;    // [M] 0.5*(w[2m], w[2m+1])
  const float2* tw_m;    // [M] exp(-2 pi i j / M)
  const float2* tw_n;    // [M] exp(-2 pi i k / N)
  const MelRow* rows;    // [n_mels] CSR rows of the filterbank
  const float* mel_w;    // [nnz] weights
  long long length;      // samples per signal
  int n_frames;          // frames per signal
  int hop;
  int pad;               // first frame's offset before sample 0
  int zpad;              // zero samples added on both sides of the signal
  int n_mels;
  int tile;              // frames per workgroup
  int tiles_per_signal;
  int pad_mode;
  float half_power;      // power / 2
  int vec_ok;            // interior frames may use paired (2-sample) loads
  int out_f16;           // 1: the output is float16
  int w16;               // mel weights in 16-byte pieces (nnz rounded up to 4 floats)
  int w_lds;             // LDS byte offset of the weights (after the exchange buffer)
};

// LDS strides of the exchange buffer (in complex values): per c and per a.
template <int C, int D>
constexpr int kLargeRowC = D + 1;  // (C unused: both strides take the shape)
template <int C, int D>
constexpr int kLargeRowA = C * (D + 1) + 1;

template <int A, int C, int D>
constexpr int kLargeThreads = C * D;

namespace {

// The A sample pairs z[B q + b] (q < A) of the frame starting at `base`
// (relative to x[0]) for pass-1 thread b: paired loads inside the signal,
// the padding index map at its edges.
template <int A, int B, typename InT>
__device__ __forceinline__ void large_frame_samples(float2 (&v)[A], const InT* x, int base, int L,
                                                    int b, int vec_ok, int zpad, int pad_mode) {
  if (vec_ok && base >= 0 && base + 2 * A * B <= L) {
#pragma unroll
    for (int q = 0; q < A; ++q) v[q] = load_pair_raw(x, base + 2 * (B * q + b));
  } else {
#pragma unroll
    for (int q = 0; q < A; ++q) {
      const int i = base + 2 * (B * q + b);
      v[q] = make_float2(padded_sample_raw(x, i, L, zpad, pad_mode),
                         padded_sample_raw(x, i + 1, L, zpad, pad_mode));
    }
  }
}

template <int A, int C, int D, typename InT, int PMODE, bool MANY>
__global__ __launch_bounds__((kLargeThreads<A, C, D>), 2) void mel_forward_large_kernel(LArgs a) {
  constexpr int B = C * D;
  constexpr int M = A * B;
  constexpr int NT = kLargeThreads<A, C, D>;
  constexpr int RC = kLargeRowC<C, D>;
  constexpr int RA = kLargeRowA<C, D>;
  constexpr int KPT = M / NT;  // split bins per thread
  static_assert(NT % 64 == 0 && M % NT == 0, "whole waves, whole bins per thread");
  static_assert((A * D) % NT == 0 || NT % (A * D) == 0, "pass-2 items");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  float2* Y = reinterpret_cast<float2*>(lds);
  float* P = reinterpret_cast<float*>(lds);  // power row, after the split

  const int tid = threadIdx.x;
  const int G = a.tile;
  const int L = static_cast<int>(a.length);
  const int tile = __builtin_amdgcn_readfirstlane(xcd_tile_order(blockIdx.x, gridDim.x));
  const int sig = tile / a.tiles_per_signal;
  const int t0 = (tile - sig * a.tiles_per_signal) * G;
  const int nvalid = min(G, a.n_frames - t0);
  const InT* x = static_cast<const InT*>(a.in) + static_cast<long long>(sig) * L;
  const long long obase = (static_cast<long long>(sig) * a.n_mels) * a.n_frames + t0;
  const float* WL = reinterpret_cast<const float*>(lds + a.w_lds);  // mel weights in LDS

  // The mel weights go to LDS once (direct global -> LDS loads, 16 bytes
  // per lane), landing while the first frame loads and transforms.
  {
    const int wave = tid >> 6, lane = tid & 63;
    for (int c = wave; c * 64 < a.w16; c += NT / 64) {
      const int q = c * 64 + lane;
      if (q < a.w16)
        __builtin_amdgcn_global_load_lds(a.mel_w + 4 * q, lds + a.w_lds + c * 1024, 16, 0, 0);
    }
  }

  // Each thread keeps its pass-1 window values and twiddles W_M^(b ka) and
  // its pass-2 twiddles W_M^(A d kc) in registers for the whole tile.  Where
  // the registers allow (D <= 16; the 32-point third pass of the other shape
  // needs them), frame f + 1's samples load while frame f is transformed.
  constexpr bool kPrefetch = D <= 16;
  constexpr bool kOneP2 = (A * D == NT);  // one pass-2 item per thread
  const int c1 = tid / D, d1 = tid - (tid / D) * D;  // pass-1 role: b = tid = D*c1 + d1
  float2 win[A], tw1[A];
  float2 tw2[kOneP2 ? C : 1];
#pragma unroll
  for (int q = 0; q < A; ++q) {
    const float2 w = a.win2[B * q + tid];
    win[q] = make_float2(w.x * kSampleScale<InT>, w.y * kSampleScale<InT>);
    tw1[q] = a.tw_m[tid * q];
  }
  if constexpr (kOneP2) {
#pragma unroll
    for (int kc = 0; kc < C; ++kc) tw2[kc] = a.tw_m[A * d1 * kc];
  }
  // this thread's filter in the mel stage, read once (MANY: more filters
  // than threads, thread t also takes t + NT, ..., their rows read per frame)
  MelRow row0{0, 0, 0, 0};
  if (tid < a.n_mels) row0 = a.rows[tid];
  // split twiddles W_N^k for k = tid + NT*j: the per-thread factor W_N^tid
  // times the wave-uniform W_N^(NT*j), read through the scalar unit
  const float2 wt = a.tw_n[tid];
  CFloat* twn_s = (CFloat*)(a.tw_n);
  const float hp = a.half_power;

  float2 nxt[kPrefetch ? A : 1];
  if constexpr (kPrefetch)
    large_frame_samples<A, B>(nxt, x, t0 * a.hop - a.pad, L, tid, a.vec_ok, a.zpad, a.pad_mode);

  for (int f = 0; f < nvalid; ++f) {
    // ---- pass 1: samples, window, A-point DFTs, twiddles ------------------
    {
      float2 v[A];
      if constexpr (kPrefetch) {
#pragma unroll
        for (int q = 0; q < A; ++q) v[q] = nxt[q];
        if (f + 1 < nvalid)
          large_frame_samples<A, B>(nxt, x, (t0 + f + 1) * a.hop - a.pad, L, tid, a.vec_ok, a.zpad,
                                    a.pad_mode);
      } else {
        large_frame_samples<A, B>(v, x, (t0 + f) * a.hop - a.pad, L, tid, a.vec_ok, a.zpad,
                                  a.pad_mode);
      }
#pragma unroll
      for (int q = 0; q < A; ++q) v[q] = make_float2(v[q].x * win[q].x, v[q].y * win[q].y);
      Dft<A>::run(v);
      float2* yp = Y + RC * c1 + d1;
      yp[0] = v[0];
#pragma unroll
      for (int ka = 1; ka < A; ++ka) yp[RA * ka] = cmul(v[ka], tw1[ka]);
    }
    __syncthreads();
    // ---- pass 2: C-point DFTs over c, twiddles W_B^(d kc) = W_M^(A d kc) ---
    for (int it = tid; it < A * D; it += NT) {
      const int ka = it / D, d = it - (it / D) * D;
      float2* yp = Y + RA * ka + d;
      float2 u[C];
#pragma unroll
      for (int c = 0; c < C; ++c) u[c] = yp[RC * c];
      Dft<C>::run(u);
      yp[0] = u[0];
#pragma unroll
      for (int kc = 1; kc < C; ++kc)
        yp[RC * kc] = cmul(u[kc], kOneP2 ? tw2[kOneP2 ? kc : 0] : a.tw_m[A * d * kc]);
    }
    __syncthreads();
    // ---- pass 3: D-point DFTs over d -------------------------------------
    for (int it = tid; it < A * C; it += NT) {
      const int ka = it / C, kc = it - (it / C) * C;
      float2* yp = Y + RA * ka + RC * kc;
      float2 s[D];
#pragma unroll
      for (int d = 0; d < D; ++d) s[d] = yp[d];
      Dft<D>::run(s);
#pragma unroll
      for (int kd = 0; kd < D; ++kd) yp[kd] = s[kd];
    }
    __syncthreads();
    // ---- real split and |X|^p: bin k = tid + NT*j and its mirror ---------
    float pw[KPT];
    float p_nyq = 0.0f;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int k = tid + NT * j;
      const int km = (M - k) & (M - 1);
      const float2 zk = Y[RA * (k % A) + RC * ((k / A) % C) + k / (A * C)];
      const float2 zm = Y[RA * (km % A) + RC * ((km / A) % C) + km / (A * C)];
      const float2 wj = make_float2(twn_s[2 * NT * j], twn_s[2 * NT * j + 1]);
      const float2 w = j == 0 ? wt : cmul(wt, wj);
      const float2 e = make_float2(zk.x + zm.x, zk.y - zm.y);  // Z[k] + conj Z[M-k]
      const float2 o = make_float2(zk.x - zm.x, zk.y + zm.y);  // Z[k] - conj Z[M-k]
      const float2 v = cmul(w, o);
      const float ax = e.x + v.y, ay = e.y - v.x;  // X[k] = e - i v
      pw[j] = power_of<PMODE>(fmaf(ax, ax, ay * ay), hp);
      if (j == 0 && tid == 0) {  // X[M] = conj(e + i v) at k = 0
        const float bx = e.x - v.y, by = e.y + v.x;
        p_nyq = power_of<PMODE>(fmaf(bx, bx, by * by), hp);
      }
    }
    __syncthreads();  // every read of the spectrum is done: P may overwrite it
#pragma unroll
    for (int j = 0; j < KPT; ++j) P[tid + NT * j] = pw[j];
    if (tid == 0) P[M] = p_nyq;
    if (f == 0) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the weight copies have landed
    __syncthreads();
    // ---- mel projection: filter m over its CSR run ------------------------
    if constexpr (!MANY) {
      if (tid < a.n_mels) {
        const float* pr = P + row0.first;
        const float* wr = WL + row0.off;
        float acc = 0.0f;
        for (int j = 0; j < row0.len; ++j) acc = fmaf(pr[j], wr[j], acc);
        const long long o = obase + static_cast<long long>(tid) * a.n_frames + f;
        if (a.out_f16) static_cast<_Float16*>(a.out)[o] = static_cast<_Float16>(acc);
        else static_cast<float*>(a.out)[o] = acc;
      }
    } else {
#pragma unroll 1
      for (int m = tid; m < a.n_mels; m += NT) {
        const MelRow row = m == tid ? row0 : a.rows[m];
        const float* pr = P + row.first;
        const float* wr = WL + row.off;
        float acc = 0.0f;
        for (int j = 0; j < row.len; ++j) acc = fmaf(pr[j], wr[j], acc);
        const long long o = obase + static_cast<long long>(m) * a.n_frames + f;
        if (a.out_f16) static_cast<_Float16*>(a.out)[o] = static_cast<_Float16>(acc);
        else static_cast<float*>(a.out)[o] = acc;
      }
    }
    __syncthreads();  // P is read before the next frame's pass 1 overwrites it
  }
}

}  // namespace

// Kernel entry of one large shape for an input type, a power mode (0: p =
// 2, 1: p = 1, 2: general p) and whether the plan has more filters than the
// workgroup has threads (built only for shapes of fewer than 256 threads;
// nullptr otherwise); instantiated in fm_large_<A>x<C>x<D>.hip.
template <int A, int C, int D>
void* large_kernel_for(int in_dtype, int pmode, bool many) {
  auto pick = [](auto in_tag, auto many_tag, int pm) -> void* {
    using InT = decltype(in_tag);
    constexpr bool M = decltype(many_tag)::value;
    if (pm == 0) return reinterpret_cast<void*>(&mel_forward_large_kernel<A, C, D, InT, 0, M>);
    if (pm == 1) return reinterpret_cast<void*>(&mel_forward_large_kernel<A, C, D, InT, 1, M>);
    return reinterpret_cast<void*>(&mel_forward_large_kernel<A, C, D, InT, 2, M>);
  };
  if (many) {
    if constexpr (kLargeThreads<A, C, D> < kMaxMels) {
      if (in_dtype == FM_I16) return pick(int16_t{}, std::true_type{}, pmode);
      return pick(float{}, std::true_type{}, pmode);
    } else {
      return nullptr;
    }
  }
  if (in_dtype == FM_I16) return pick(int16_t{}, std::false_type{}, pmode);
  return pick(float{}, std::false_type{}, pmode);
}

// Large shapes built into the library (n_fft/2 = A * C * D).
#define FM_FOR_EACH_LARGE_SHAPE(X) X(16, 16, 8) X(16, 16, 16) X(16, 16, 32)
#define FM_DECLARE_LARGE_SHAPE(A, C, D) extern template void* large_kernel_for<A, C, D>(int, int, bool);
FM_FOR_EACH_LARGE_SHAPE(FM_DECLARE_LARGE_SHAPE)
#undef FM_DECLARE_LARGE_SHAPE

}  // namespace fm
