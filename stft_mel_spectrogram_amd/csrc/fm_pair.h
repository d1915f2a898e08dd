// Paired-frame, software-pipelined mel-spectrogram forward kernel for gfx950
// (MI355X): device code.  fm_pair_<R>x<R>.hip instantiates it; fm_launch.hip
// chooses it per plan (fm_forward's default for the shapes it is built for).
//
// The chain is the one the flashmel 0.1.0 page describes (README "How it
// works": padding as index arithmetic, window, real FFT, |X|^power, sparse
// mel projection, one launch).  Two things differ from fm_kernel.h:
//
// * Two real frames a and b of one signal go through ONE complex FFT of
//   n_fft = R*R points, z[n] = a[n] + i b[n] (the pages name this packing;
//   README "How it works", R2C modes).  With Z = FFT(z),
//       A[k] = (Z[k] + conj Z[N-k]) / 2,   B[k] = (Z[k] - conj Z[N-k]) / (2i)
//   are the two frames' spectra, so |A|^2 and |B|^2 cost four additions and
//   four multiply-adds per bin for both frames (the window is pre-scaled by
//   1/2).  The FFT is Cooley-Tukey R x R with one LDS exchange:
//     pass 1, thread (column n2, pair): R-point DFT over n1 of z[R*n1 + n2],
//             times exp(-2 pi i n2 k1 / N), stored Y[pair][k1][n2];
//     pass 2, thread (row k1, pair): R-point DFT over n2 of row k1, giving
//             Z[k1 + R*k2]; the upper half of the row goes back to LDS, and
//             every thread then reads the mirrored bins N-k of its own lower
//             half from the row R-k1 (row 0 mirrors into itself).
//   Both passes have R threads per frame pair, so a 256-thread workgroup
//   keeps nearly every lane busy in both.  The R-point DFTs are
//   register-resident (R = 20: Good-Thomas 4 x 5, no inner twiddles).
//
// * The workgroup is persistent: it owns a contiguous range of frames (of
//   the flattened batch x frames space) and walks it in chunks of up to
//   2*floor(256/R) frames.  The samples of chunk c+1 are loaded into
//   registers (16-byte loads of the chunk's contiguous sample span, or, for
//   chunks that reach into the padding, one padded sample at a time) while
//   chunk c is transformed, and written to an LDS span buffer when chunk c
//   is done; so HBM reads, the FFT's VALU work, the mel stage's matrix-core
//   work and the output stores of different chunks overlap.
#pragma once

#include "fm_kernel.h"

namespace fm {

// Kernel arguments of the paired kernel (one struct, passed by value).
struct PArgs {
  const void* in;          // [B, L] float32 or int16
  void* out;               // [B, n_mels, n_frames] float32 or float16
  const float* win;        // [n_fft] window * 1/2
  const float2* tw_n;      // [n_fft/2] exp(-2 pi i k / n_fft)
  const int* mel_tbl;      // as KArgs::mel_tbl
  const float* blk_w;      // block weights (w_floats of them, a multiple of 256)
  long long length;        // samples per signal
  long long in_elems;      // batch * length: the input allocation, in samples
  long long total;         // batch * n_frames
  int n_frames;
  int hop;
  int pad;                 // first frame's offset before sample 0
  int zpad;                // zero samples added on both sides
  int pad_mode;
  int n_mels;
  int chunk;               // frames per chunk at most (even)
  int w_floats;
  int out_f16;
  float half_power;
  int span_lds;            // LDS byte offset of the sample span buffer (later
                           // the power tile)
  int w_lds;               // LDS float offset of the mel weights
};

// Most samples a chunk's span may hold (frames' extent plus the 16-byte
// alignment slack of the interior loads); the host sizes chunks to fit.
constexpr int kPairSpanFloats = 4096;
constexpr int kPairThreads = 256;
// Row pitch (floats) of the output tile: >= 32 frames, = 4 mod 16.
constexpr int kPairOutPitch = 36;

namespace {

// Mel projection of one chunk (nv <= 32 frames) for one wave's blocks, as
// mel_blocks in fm_kernel.h (16 filters x 16 frames x 4 bins per
// v_mfma_f32_16x16x4f32, weights and power tile in LDS).  The results go to
// the chunk's output tile O[filter][frame] in LDS (row pitch kPairOutPitch):
// they are stored to HBM at the start of the next chunk, after that chunk's
// samples have arrived, so that waiting for sample loads never waits for
// output stores (one wave's loads and stores share a completion counter).
template <int KS, int NFB>
__device__ __forceinline__ void pair_mel(const float* P, const float* WL, float* O, int nv, int lane,
                                         CInt* blk, int bb, int be) {
  constexpr int U = kMelStepGroup;
  const int fr = lane & 15, kq = lane >> 4;
  int roff[NFB];
#pragma unroll
  for (int f = 0; f < NFB; ++f) roff[f] = min(16 * f + fr, nv - 1) * KS + kq;
  for (int bi = bb; bi < be; ++bi) {
    const int kb = blk[4 * bi], ks = blk[4 * bi + 1] & 1023, woff = blk[4 * bi + 2];
    const int mel0 = blk[4 * bi + 3] & 0xffff, nrow = blk[4 * bi + 3] >> 16;  // mel_filter_word
    f32x4 acc[NFB];
#pragma unroll
    for (int f = 0; f < NFB; ++f) acc[f] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const float* pb = P + kb;
    const float* wl = WL + woff + lane;
    for (int s0 = 0; s0 < ks; s0 += U, pb += 4 * U, wl += 64 * U) {
      float av[U], bv[U][NFB];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        av[u] = wl[64 * u];
#pragma unroll
        for (int f = 0; f < NFB; ++f) bv[u][f] = pb[roff[f] + 4 * u];
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int f = 0; f < NFB; ++f)
          acc[f] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], bv[u][f], acc[f], 0, 0, 0);
    }
    // lane (fr, kq) holds filters mel0 + 4 kq + r of frame 16 f + fr; with
    // the pitch at 4 mod 16 rows the 64 lanes' writes hit distinct banks
    float* orow = O + (mel0 + 4 * kq) * kPairOutPitch + fr;
#pragma unroll
    for (int f = 0; f < NFB; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * kq + r < nrow) orow[r * kPairOutPitch + 16 * f] = acc[f][r];  // (the block's own filters only)
  }
}

// One chunk: signal b, frames t0 .. t0+nv-1.
struct PairChunk {
  int b, t0, nv;
};

}  // namespace

template <int R, typename InT, int PMODE>
__global__ __launch_bounds__(kPairThreads, 2) void mel_pair_kernel(PArgs a) {
  constexpr int NF = R * R;           // n_fft
  constexpr int HALF = NF / 2;        // bins 0..HALF
  constexpr int SY = NF + 4;          // pair stride of the exchange buffer (complex)
  constexpr int SP = power_stride(HALF);  // frame stride of the power tile (odd)
  constexpr int NT = kPairThreads;
  constexpr int MAXP = NT / R;        // frame pairs per chunk
  constexpr int H = R / 2;            // bins per row task below the mirror line
  constexpr int ES = static_cast<int>(sizeof(InT));
  constexpr int SPAN_PER_THREAD = kPairSpanFloats / NT;  // padded-path samples per thread
  static_assert(R % 2 == 0, "rows pair up around R/2");
  static_assert(SPAN_PER_THREAD % 4 == 0, "padded-path samples are held as float4");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  float2* Y = reinterpret_cast<float2*>(lds);
  float* span = reinterpret_cast<float*>(lds + a.span_lds);
  float* P = span;  // power tile, in the span buffer (free after pass 1)
  float* WL = reinterpret_cast<float*>(lds) + a.w_lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = tid % R;   // pass 1: column n2; pass 2: row k1
  const int pr = tid / R;    // frame pair within the chunk
  const bool act = pr < MAXP;
  const int L = static_cast<int>(a.length);
  const int T = a.n_frames;
  const int hop = a.hop;

  float wv[R];   // window at this column's samples, R*n1 + col
  float2 tv[R];  // exp(-2 pi i col k1 / N)
  // ---- this workgroup's frames: [F0, F1) of the batch x frames space ----
  const int vwg = xcd_tile_order(blockIdx.x, gridDim.x);
  const long long F0 = static_cast<long long>(vwg) * a.total / gridDim.x;
  const long long F1 = static_cast<long long>(vwg + 1) * a.total / gridDim.x;

  // The next chunk from frame f: within one signal, the remaining frames of
  // the signal segment split evenly into chunks of at most a.chunk (even
  // sizes where possible, so frame pairs are full).
  auto chunk_at = [&](long long f) {
    PairChunk c;
    const long long bl = f / T;
    c.b = static_cast<int>(bl);
    c.t0 = static_cast<int>(f - bl * T);
    const long long seg_l = min(F1 - f, static_cast<long long>(T - c.t0));
    const int seg = static_cast<int>(seg_l);
    const int n = (seg + a.chunk - 1) / a.chunk;
    int nv = (seg + n - 1) / n;
    if ((nv & 1) && nv < seg) ++nv;
    c.nv = nv;
    return c;
  };

  // ---- prefetch of a chunk's samples into registers ----
  // interior chunks: the 16-byte-aligned byte range around the chunk's
  // samples, one 16-byte piece per thread and round (q = tid + NT*i);
  // chunks reaching into the padding: sample s = tid + NT*i of the span
  // through the padding index map, in pre[i/4] component i%4.
  float4 pre[SPAN_PER_THREAD / 4];
  auto prefetch = [&](const PairChunk& c, bool& interior, int& off0, int& n16) {
    const long long s0 = static_cast<long long>(c.t0) * hop - a.pad;  // first sample
    const int len = (c.nv - 1) * hop + NF;
    const InT* x = static_cast<const InT*>(a.in) + static_cast<long long>(c.b) * L;
    const uintptr_t xa = reinterpret_cast<uintptr_t>(a.in);
    const uintptr_t xe = xa + static_cast<uintptr_t>(a.in_elems) * ES;
    const uintptr_t lo = reinterpret_cast<uintptr_t>(x) + static_cast<uintptr_t>(s0 * ES);
    const uintptr_t g_lo = lo & ~static_cast<uintptr_t>(15);
    const uintptr_t g_hi = (lo + static_cast<uintptr_t>(len) * ES + 15) & ~static_cast<uintptr_t>(15);
    interior = s0 >= 0 && s0 + len <= L && g_lo >= xa && g_hi <= xe && (lo % ES) == 0;
    if (interior) {
      off0 = static_cast<int>((lo - g_lo) / ES);
      n16 = static_cast<int>((g_hi - g_lo) >> 4);
#pragma unroll
      for (int i = 0; i < SPAN_PER_THREAD / 4; ++i) {
        const int q = tid + NT * i;
        if (q < n16) pre[i] = *reinterpret_cast<const float4*>(g_lo + 16 * static_cast<uintptr_t>(q));
      }
    } else {
      off0 = 0;
      n16 = 0;
      const int s0i = static_cast<int>(s0);
#pragma unroll
      for (int i = 0; i < SPAN_PER_THREAD; ++i) {
        const int s = tid + NT * i;
        float v = 0.0f;
        if (s < len) v = padded_sample_raw(x, s0i + s, L, a.zpad, a.pad_mode);
        if ((i & 3) == 0) pre[i >> 2].x = v;
        if ((i & 3) == 1) pre[i >> 2].y = v;
        if ((i & 3) == 2) pre[i >> 2].z = v;
        if ((i & 3) == 3) pre[i >> 2].w = v;
      }
    }
  };
  // Registers -> LDS span (float32; int16 converted, unscaled).
  auto stage_span = [&](bool interior, int n16, int len) {
    if (interior) {
      if constexpr (std::is_same<InT, float>::value) {
#pragma unroll
        for (int i = 0; i < SPAN_PER_THREAD / 4; ++i) {
          const int q = tid + NT * i;
          if (q < n16) *reinterpret_cast<float4*>(span + 4 * q) = pre[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < SPAN_PER_THREAD / 4; ++i) {
          const int q = tid + NT * i;
          if (q < n16) {
            const unsigned w[4] = {__float_as_uint(pre[i].x), __float_as_uint(pre[i].y),
                                   __float_as_uint(pre[i].z), __float_as_uint(pre[i].w)};
            float f[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              f[2 * e] = static_cast<float>(static_cast<short>(w[e] & 0xFFFFu));
              f[2 * e + 1] = static_cast<float>(static_cast<short>(w[e] >> 16));
            }
            *reinterpret_cast<float4*>(span + 8 * q) = make_float4(f[0], f[1], f[2], f[3]);
            *reinterpret_cast<float4*>(span + 8 * q + 4) = make_float4(f[4], f[5], f[6], f[7]);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < SPAN_PER_THREAD; ++i) {
        const int s = tid + NT * i;
        const float v = (i & 3) == 0 ? pre[i >> 2].x : (i & 3) == 1 ? pre[i >> 2].y
                        : (i & 3) == 2 ? pre[i >> 2].z : pre[i >> 2].w;
        if (s < len) span[s] = v;
      }
    }
  };

  CInt* tbl = (CInt*)(a.mel_tbl);
  const int bb = tbl[wave], be = tbl[wave + 1];
  CInt* blk = tbl + 8;
  float* O = reinterpret_cast<float*>(lds);  // output tile, in the exchange buffer's bytes
  // The output tile of a chunk -> HBM, frames contiguous: lanes 0-31 one
  // filter row's frames, lanes 32-63 the next row's; streaming stores.
  auto store_tile = [&](const PairChunk& c) {
    const int oc = tid & 31;
    if (oc < c.nv) {
      const long long obase = (static_cast<long long>(c.b) * a.n_mels) * T + c.t0 + oc;
      for (int m = tid >> 5; m < a.n_mels; m += NT / 32) {
        const float v = O[m * kPairOutPitch + oc];
        if (a.out_f16)
          __builtin_nontemporal_store(static_cast<_Float16>(v),
                                      static_cast<_Float16*>(a.out) + obase + static_cast<long long>(m) * T);
        else
          __builtin_nontemporal_store(v, static_cast<float*>(a.out) + obase + static_cast<long long>(m) * T);
      }
    }
  };

  long long f = F0;
  PairChunk cur{0, 0, 0}, prev{0, 0, 0};
  bool have_prev = false;
  bool interior = false;
  int off0 = 0, n16 = 0;
  // The first chunk's samples are requested before anything else.
  if (f < F1) {
    cur = chunk_at(f);
    prefetch(cur, interior, off0, n16);
  }
  // ---- tables, once per workgroup: the window and the twiddles
  //      exp(-2 pi i k / N) land in LDS with 16-byte loads (in the exchange
  //      buffer, free until the first chunk's pass 1), the mel block weights
  //      behind the span buffer; then every thread takes the window at its
  //      column's samples and the twiddles exp(-2 pi i n2 k1 / N) of its
  //      outputs into registers ----
  {
    float* tw_l = reinterpret_cast<float*>(lds);  // [N] floats: exp(-2 pi i k/N), k < N/2
    float* win_l = tw_l + NF;                     // [N] window * 1/2
    constexpr int NQ = NF / 4;                    // float4 per table
    float4 tq;
    if (tid < 2 * NQ)
      tq = tid < NQ ? reinterpret_cast<const float4*>(a.tw_n)[tid]
                    : reinterpret_cast<const float4*>(a.win)[tid - NQ];
    for (int i = 4 * tid; i < a.w_floats; i += 4 * NT)
      *reinterpret_cast<float4*>(WL + i) = *reinterpret_cast<const float4*>(a.blk_w + i);
    if (tid < 2 * NQ) reinterpret_cast<float4*>(tw_l)[tid] = tq;
    __syncthreads();
#pragma unroll
    for (int n1 = 0; n1 < R; ++n1) wv[n1] = win_l[R * n1 + col] * kSampleScale<InT>;
#pragma unroll
    for (int k1 = 0; k1 < R; ++k1) {
      const int e = col * k1;  // < N
      const float2 t = reinterpret_cast<const float2*>(tw_l)[e < HALF ? e : e - HALF];
      tv[k1] = e < HALF ? t : make_float2(-t.x, -t.y);
    }
  }
  while (f < F1) {
    const int nv = cur.nv;
    const int npairs = (nv + 1) >> 1;
    __syncthreads();  // the previous chunk's output tile is complete; its power tile is read
    // this chunk's samples: registers -> LDS span (waits for their loads)
    stage_span(interior, n16, (nv - 1) * hop + NF);
    const int coff = off0;
    // the previous chunk's output leaves now, after this chunk's samples
    // have arrived and before the next chunk's loads are issued
    if (have_prev) store_tile(prev);
    __syncthreads();  // span visible; the output tile is read, the exchange buffer free

    // ---- pass 1: window, R-point DFT over n1, twiddle -> Y[pair][k1][n2] ----
    const bool p1 = act && pr < npairs;
    // pair pr = frames pr and pr + npairs (a lone last frame pairs with
    // itself); frames hop apart start on banks that differ, so the lanes of
    // a wave's pairs collide less than with neighbouring frames
    const int fa = pr, fb_raw = pr + npairs, fb = min(fb_raw, nv - 1);
    if (p1) {
      const float* sa = span + coff + fa * hop + col;
      const float* sb = span + coff + fb * hop + col;
      float2 v[R];
#pragma unroll
      for (int n1 = 0; n1 < R; ++n1) v[n1] = make_float2(sa[R * n1] * wv[n1], sb[R * n1] * wv[n1]);
      Dft<R>::run(v);
      float2* yc = Y + pr * SY + col;
      yc[0] = v[0];
#pragma unroll
      for (int k1 = 1; k1 < R; ++k1) yc[R * k1] = cmul(v[k1], tv[k1]);
    }
    // the next chunk's samples load while this one is transformed
    const long long fn = f + nv;
    PairChunk nxt{0, 0, 0};
    bool n_interior = false;
    int n_off0 = 0, n_n16 = 0;
    if (fn < F1) {
      nxt = chunk_at(fn);
      prefetch(nxt, n_interior, n_off0, n_n16);
    }
    __syncthreads();

    // ---- pass 2: R-point DFT of row k1 = col; upper half back to LDS ----
    float2 z[R];
    if (p1) {
      float2* yr = Y + pr * SY + R * col;
#pragma unroll
      for (int n2 = 0; n2 < R; ++n2) z[n2] = yr[n2];
      Dft<R>::run(z);
#pragma unroll
      for (int k2 = H; k2 < R; ++k2) yr[k2] = z[k2];
    }
    __syncthreads();
    // ---- separation: bins k = col + R*k2 (k2 < H, and N/2 for row 0) of
    //      both frames from Z[k] and Z[N-k], straight into the power tile ----
    if (p1) {
      // mirror of (k1, k2) is (R-k1, R-1-k2); for k1 = 0 it is (0, R-k2),
      // and (0, 0) for k2 = 0
      const int mrow = (R - col) % R;
      const float2* ym = Y + pr * SY + R * mrow + (R - 1) + (col == 0 ? 1 : 0);
      const float hp = a.half_power;
      float* qa = P + fa * SP + col;
      float* qb = P + fb * SP + col;
      const bool wb = fb_raw < nv;
#pragma unroll
      for (int k2 = 0; k2 < H; ++k2) {
        float2 zm = ym[-k2];
        if (k2 == 0 && col == 0) zm = z[0];
        const float2 zk = z[k2];
        const float s1 = zk.x + zm.x, d1 = zk.y - zm.y;  // 2 A[k] (window carries 1/2)
        const float s2 = zk.y + zm.y, d2 = zk.x - zm.x;  // |2 B[k]| from (d2, s2)
        qa[R * k2] = power_of<PMODE>(fmaf(s1, s1, d1 * d1), hp);
        if (wb) qb[R * k2] = power_of<PMODE>(fmaf(s2, s2, d2 * d2), hp);
      }
      if (col == 0) {  // bin N/2 (row 0, k2 = H) mirrors into itself
        const float2 zk = z[H];
        qa[HALF] = power_of<PMODE>(4.0f * zk.x * zk.x, hp);
        if (wb) qb[HALF] = power_of<PMODE>(4.0f * zk.y * zk.y, hp);
      }
    }
    // the mel stage reads up to kMelTileOverrun - 1 floats past the last
    // frame's row: keep them 0 (no frame's row is there)
    if (tid < kMelTileOverrun) P[nv * SP + tid] = 0.0f;
    __syncthreads();

    // ---- mel projection on the matrix cores into the output tile ----
    if (nv > 16) pair_mel<SP, 2>(P, WL, O, nv, lane, blk, bb, be);
    else pair_mel<SP, 1>(P, WL, O, nv, lane, blk, bb, be);

    prev = cur;
    have_prev = true;
    f = fn;
    cur = nxt;
    interior = n_interior;
    off0 = n_off0;
    n16 = n_n16;
  }
  if (have_prev) {
    __syncthreads();
    store_tile(prev);
  }
}

// Kernel entry for an input type and power mode (0: p = 2, 1: p = 1,
// 2: general p); instantiated in fm_pair_<R>x<R>.hip.
template <int R>
void* pair_kernel_for(int in_dtype, int pmode) {
  if (in_dtype == FM_I16) {
    if (pmode == 0) return reinterpret_cast<void*>(&mel_pair_kernel<R, int16_t, 0>);
    if (pmode == 1) return reinterpret_cast<void*>(&mel_pair_kernel<R, int16_t, 1>);
    return reinterpret_cast<void*>(&mel_pair_kernel<R, int16_t, 2>);
  }
  if (pmode == 0) return reinterpret_cast<void*>(&mel_pair_kernel<R, float, 0>);
  if (pmode == 1) return reinterpret_cast<void*>(&mel_pair_kernel<R, float, 1>);
  return reinterpret_cast<void*>(&mel_pair_kernel<R, float, 2>);
}

extern template void* pair_kernel_for<20>(int, int);

}  // namespace fm
