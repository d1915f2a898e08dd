// Row-per-thread forward kernel for the FFT shapes with N1 = 8 (n_fft =
// 16 * N2) on gfx950: device code.  Same chain, tables, tile layout and mel
// stage as fm_kernel.h; what differs is how the work is cut:
//
// * 512 threads (8 waves) per tile instead of 256, so a pass-1 round covers
//   floor(512 / N2) frames and a thread loads and transforms fewer frames;
// * the second pass gives every row k1 of a frame its own thread (8 per
//   frame) instead of every pair of mirrored rows: a thread runs one
//   N2-point DFT instead of two, then half of the real split of its row
//   pair.  The split of bin k = k1 + 8 k2 needs Z[M - k], which lies in row
//   8 - k1 (the same row for k1 = 0 and 4): the 8 threads of a frame are 8
//   consecutive lanes of one wave, so the partner row's values come over
//   lane permutes (ds_bpermute), not through LDS.  Thread k1 < 4 takes the
//   pairs k2 = 0 .. (N2-1)/2 of rows k1 and 8-k1 (rows 0 and 4 pair with
//   themselves), thread k1 > 4 the remaining (N2-1)/2 of its row pair.
//
// Each thread's dependent chain in the second pass is about half as long
// as in fm_kernel.h's, at the same amount of work per frame.
#pragma once

#include "fm_kernel.h"

namespace fm {

constexpr int kRowsThreads = 512;

namespace {

__device__ __forceinline__ float lane_fetch(int src_lane_bytes, float v) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane_bytes, __float_as_int(v)));
}

template <int N2, typename InT, int PMODE>
__global__ __launch_bounds__(kRowsThreads, 4) void mel_forward_rows_kernel(KArgs a) {
  constexpr int N1 = 8;
  constexpr int M = N1 * N2;
  constexpr int NF = 2 * M;
  constexpr int RS = exchange_row(N2);
  constexpr int SY = exchange_stride(N1, N2);
  constexpr int SP = power_stride(M);
  constexpr int NT = kRowsThreads;
  constexpr int NW = NT / 64;
  constexpr int SLOTS = NT / N2;               // frames per pass-1 round
  constexpr int RMAX = (64 + SLOTS - 1) / SLOTS;
  constexpr int CP = (N2 + 1) / 2;             // split pairs of a thread k1 < 4 (and rows 0, 4)
  static_assert(N2 % 2 == 1, "odd rows: rows 0 and 4 pair within themselves without a middle bin");
  static_assert(M <= 256, "split twiddles kept in registers");
  static_assert(power_stride(M) == M + 1, "power rows without a pad to clear");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  float2* Y = reinterpret_cast<float2*>(lds);  // Y[f][k1][n2]
  float* P = reinterpret_cast<float*>(lds);    // P[f][k], aliases Y

  const int tid = threadIdx.x;
  const int G = a.tile;
  const int L = static_cast<int>(a.length);
  const int n2 = tid % N2;     // pass-1 role
  const int slot = tid / N2;
  const int f2 = tid >> 3;     // pass-2 role: frame f2, row k1
  const int k1 = tid & 7;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  const int tile = __builtin_amdgcn_readfirstlane(xcd_tile_order(blockIdx.x, gridDim.x));
  const int b = tile / a.tiles_per_signal;
  const int t0 = (tile - b * a.tiles_per_signal) * G;
  const int nvalid = min(G, a.n_frames - t0);
  const InT* x = static_cast<const InT*>(a.in) + static_cast<long long>(b) * L;

  // ---- pass 1: window + 8-point DFTs, twiddle, exchange through LDS -------
  const bool p1 = slot < SLOTS;
  {
    float2 win[N1], twv[N1];
#pragma unroll
    for (int n1 = 0; n1 < N1; ++n1) {
      const float2 w = a.win2[N2 * n1 + n2];
      win[n1] = make_float2(w.x * kSampleScale<InT>, w.y * kSampleScale<InT>);
    }
    twv[0] = make_float2(1.0f, 0.0f);
#pragma unroll
    for (int q = 1; q < N1; ++q) twv[q] = a.tw_m[N2 * q + n2];
    float2 sb[RMAX][N1];
    if (p1) {
#pragma unroll
      for (int r = 0; r < RMAX; ++r) {
        const int f = slot + SLOTS * r;
        if (f < nvalid) {
          const int base = (t0 + f) * a.hop - a.pad;
          if (a.vec_ok && base >= 0 && base + NF <= L) {  // interior frame
#pragma unroll
            for (int n1 = 0; n1 < N1; ++n1) sb[r][n1] = load_pair_raw(x, base + 2 * (N2 * n1 + n2));
          } else {
#pragma unroll
            for (int n1 = 0; n1 < N1; ++n1) {
              const int i = base + 2 * (N2 * n1 + n2);
              sb[r][n1] = make_float2(padded_sample_raw(x, i, L, a.zpad, a.pad_mode),
                                      padded_sample_raw(x, i + 1, L, a.zpad, a.pad_mode));
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < RMAX; ++r) {
        const int f = slot + SLOTS * r;
        if (f < nvalid) {
          float2 v[N1];
#pragma unroll
          for (int n1 = 0; n1 < N1; ++n1) v[n1] = make_float2(sb[r][n1].x * win[n1].x, sb[r][n1].y * win[n1].y);
          Dft<N1>::run(v);
          float2* yrow = Y + f * SY + n2;
          yrow[0] = v[0];
#pragma unroll
          for (int q = 1; q < N1; ++q) yrow[q * RS] = cmul(v[q], twv[q]);
        }
      }
    }
  }
  __syncthreads();

  // ---- pass 2: one N2-point DFT per thread (frame f2, row k1) ------------
  const bool has = f2 < nvalid;
  float2 za[N2], wv[CP];
  if (has) {
#pragma unroll
    for (int j = 0; j < CP; ++j) wv[j] = a.tw_n[k1 + N1 * j];  // split twiddles, under the DFT
    const float2* ra = Y + f2 * SY + k1 * RS;
#pragma unroll
    for (int j = 0; j < N2; ++j) za[j] = ra[j];
    Dft<N2>::run(za);
  }
  // the partner row 8 - k1 (k1 = 0, 4: the row itself) of the same frame,
  // mirrored: pv[j] = Z_partner[N2 - 1 - j], j < CP (all lanes take part)
  const int partner = ((lane & ~7) | ((N1 - k1) & 7)) * 4;
  float2 pv[CP];
#pragma unroll
  for (int j = 0; j < CP; ++j)
    pv[j] = make_float2(lane_fetch(partner, za[N2 - 1 - j].x), lane_fetch(partner, za[N2 - 1 - j].y));
  __syncthreads();  // every read of the exchange buffer is done: P may overwrite it
  // Every read of the exchange buffer is done: stream the mel weights into
  // LDS behind the power tile, landing while the split runs.
  for (int c = wave; c < a.w_chunks; c += NW)
    __builtin_amdgcn_global_load_lds(a.blk_w + c * 256 + lane * 4, P + a.w_lds + c * 256, 16, 0, 0);
  if (tid < kMelTileOverrun) P[nvalid * SP + tid] = 0.0f;  // what the mel stage may read past
  if (has) {
    float* prow = P + f2 * SP;
    const float hp = a.half_power;
    const bool r0 = (k1 == 0);
#pragma unroll
    for (int j = 0; j < CP; ++j) {
      // bin k = k1 + 8 j and its mirror M - k: row 0 pairs k2 with
      // (N2 - k2) mod N2, i.e. the mirrored value one step back
      const float2 zm = r0 ? (j == 0 ? za[0] : pv[j - 1]) : pv[j];
      if (j < CP - 1 || k1 < 5)  // the last pair of rows 5..7 belongs to rows 3..1
        split_pair<PMODE>(prow + k1 + N1 * j, prow + (M - k1 - N1 * j), za[j], zm, wv[j], hp);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // the weight copies have landed in LDS
  __syncthreads();

  // ---- mel projection on the matrix cores (fm_kernel.h's mel_blocks) -----
  {
    CInt* tbl = (CInt*)(a.mel_tbl);
    const int bb = wave < kMelWaves ? tbl[wave] : 0, be = wave < kMelWaves ? tbl[wave + 1] : 0;
    const long long obase = static_cast<long long>(b) * a.n_mels * a.n_frames + t0;
    const int nfb = (G + 15) >> 4;
    CInt* blk = tbl + 8;
    const float* WL = P + a.w_lds;
    float* stg = P + a.w_lds + a.w_chunks * 256 + (wave < kMelWaves ? wave : 0) * kMelStageFloats;
    switch (nfb) {
#define FM_MEL_CALL(NFB, STAGE)                                                                \
  if (a.out_f16)                                                                              \
    mel_blocks<SP, NFB, STAGE, false, _Float16>(P, WL, stg, G, nvalid, lane,                   \
                                            static_cast<_Float16*>(a.out) + obase, a.n_frames, \
                                            a.n_mels, blk, bb, be);                           \
  else                                                                                        \
    mel_blocks<SP, NFB, STAGE, false, float>(P, WL, stg, G, nvalid, lane,                     \
                                         static_cast<float*>(a.out) + obase, a.n_frames,      \
                                         a.n_mels, blk, bb, be)
      case 1: FM_MEL_CALL(1, false); break;
      case 2: FM_MEL_CALL(2, false); break;
      case 3: FM_MEL_CALL(3, true); break;
      default: FM_MEL_CALL(4, true); break;
#undef FM_MEL_CALL
    }
  }
}

}  // namespace

// Kernel entry for an input type and a power mode; instantiated for N2 in
// fm_shape_8x<N2>.hip.
template <int N2>
void* rows_kernel_for(int in_dtype, int pmode) {
  auto pick = [](auto in_tag, int pm) -> void* {
    using InT = decltype(in_tag);
    if (pm == 0) return reinterpret_cast<void*>(&mel_forward_rows_kernel<N2, InT, 0>);
    if (pm == 1) return reinterpret_cast<void*>(&mel_forward_rows_kernel<N2, InT, 1>);
    return reinterpret_cast<void*>(&mel_forward_rows_kernel<N2, InT, 2>);
  };
  if (in_dtype == FM_I16) return pick(int16_t{}, pmode);
  return pick(float{}, pmode);
}

extern template void* rows_kernel_for<25>(int, int);

}  // namespace fm
