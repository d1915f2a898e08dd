// Internal declarations shared by the host plan builder, the C ABI and the
// HIP kernels of the fused mel-spectrogram forward pass.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "fm.h"

namespace fm {

// Per-mel CSR row: first bin of the contiguous support, number of bins,
// offset of its first weight in the packed weight array.
struct MelRow {
  int32_t first, len, off, pad_;
};

// The mel projection runs on the matrix cores: filters in blocks of 16 (the
// M side of a 16x16x4 f32 MFMA), each block against the contiguous run of
// bins its filters touch, in steps of 4 bins (the K side), frames as the N
// side.  A block's weights are stored dense, 64 per step, in the lane order
// of the MFMA's A operand (lane l: filter mel0 + l%16, bin kb + 4*step + l/16),
// zero where a filter has no weight.
struct MelBlock {
  int32_t kb;      // first bin of the run
  int32_t ksteps;  // 4-bin steps, a multiple of kMelStepGroup (0 when every
                   // filter of the block is empty)
  int32_t w_off;   // offset of the block's weights (floats)
  int32_t mel0;    // first filter of the block
  int32_t s_hi = 0; // steps from s_hi on hold only zero weights
  int32_t nrow = 16; // filters mel0 .. mel0 + nrow - 1 (<= 16; lanes past them hold zero weights)
};
// A block's filter word in the device table: mel0, and its filter count in
// bits 16 and up (mel0 < 256).
constexpr int32_t mel_filter_word(int mel0, int nrow) { return mel0 | (nrow << 16); }
// A block's step word in the device table: ksteps, and s_hi in bits 20 and
// up (the kernel may skip the products of the steps from s_hi on).  ksteps
// <= (n_fft/2 + 1 + 3)/4 + 3 <= 516 for n_fft <= 4096: ten bits.
constexpr int32_t mel_step_word(int ksteps, int s_hi) { return ksteps | (s_hi << 20); }
constexpr int kMelBlock = 16;
constexpr int kMaxMels = 256;      // filters per plan at most
constexpr int kMaxMelBlocks = 16;  // n_mels <= 256
constexpr int kMelWaves = 4;       // waves of a workgroup
// The kernel runs steps in groups of this many (blocks are zero-padded to
// whole groups, so the table is a whole number of 256-float chunks, the unit
// in which it is copied to LDS).
constexpr int kMelStepGroup = 4;
// Power-tile floats the mel stage may read past the tile (zeroed there).
constexpr int kMelTileOverrun = 16;
// FFTs of n_fft/2 >= this many points keep the mel weights in global memory
// (L2) instead of LDS: their weights (about n_fft/2 x 64 bytes) would force
// the tile below the geometric maximum.  The kernel then loads the weights
// in chunks of kMelGlobalChunk steps and the table carries one chunk of zero
// slack at its end.
constexpr int kMelGlobalWeightsFrom = 2048;
constexpr int kMelGlobalChunk = 32;

// Pass-1 tables (the window pairs and the twiddles exp(-2 pi i n2 k1 / M),
// 16*M bytes) of shapes that cannot hold them in registers (N1 > 8) are
// either read from global memory per frame or copied into LDS behind the
// exchange buffer at the start.  Measured: the copy pays for N1 = 16
// (n_fft 512: two pass-1 rounds per thread at 2 workgroups per CU, 22.0 ->
// 20.4 us on asr512) and for n_fft 2048 with 8-wave workgroups (every
// thread's 63 table reads per frame from L2 otherwise; 64 x 220500 samples:
// 127.7 -> 112.8 us, while either change alone gains nothing); it costs for
// n_fft 1024 (one round per thread: 13.6 -> 14.8 us).
constexpr bool tables_in_lds(int n1, int m) {
  return (n1 == 16 || (n1 == 32 && m == 1024)) && m < kMelGlobalWeightsFrom;
}
// Tiles of more than this many frames write their mel rows through a
// per-wave LDS staging area (one contiguous store per row, rows long enough
// to cover whole cache lines); narrower tiles store the MFMA results directly.
constexpr int kMelStageMinFrames = 33;
// Tiles of at least this many frames project on the vector units instead
// (mel_valu in fm_kernel.h; Plan::mel_valu): one frame per lane, the filters
// in quads of 4 consecutive filters, each quad's runs padded to its longest
// run, weights read as scalars.  Quads are cut into kMelShares contiguous
// shares of about equal cost; a workgroup of w waves gives each wave 8/w
// shares.  The threshold is measured (same box, us per launch, against the
// matrix-core blocks): n_fft 400, 8 x 480000 (47-frame tiles): 14.5 against
// 15.9; 4 x 480000 (24 frames): 12.1 against 13.4; n_fft 256, 8 x 480000:
// 21.0 against 22.1.  Below 17 frames half a wave's lanes or more idle, and
// the wider filters of the larger FFTs lose (n_fft 2048, 16-frame tiles:
// 97.6 against 83.7; n_fft 400, 1 x 480000, 12 frames: 8.4 against 7.6).
constexpr int kMelValuMinFrames = 17;
constexpr int kMelShares = 8;
constexpr int kQuadHdr = 8;  // int32 per quad: 4 start bins, run length, weight offset (float4s), 2 pad
// Staging floats per wave: 16 filters x (64 frames + 1 pad).
constexpr int kMelStageFloats = 16 * 65;
// Staging floats of a wide tile of `frames` frames, all waves: the pair
// layout stages on its kMelWaves mel waves; the row layout spreads the mel
// blocks over its 8 waves, each staging 16 filters x (16 nfb + 1) floats for
// the tile's nfb 16-frame column groups.
constexpr long mel_stage_floats(bool rows, int frames) {
  return frames < kMelStageMinFrames ? 0
         : rows ? 8L * 16 * (16 * ((frames + 15) / 16) + 1)
                : static_cast<long>(kMelWaves) * kMelStageFloats;
}

// LDS strides of a tile, padded against bank conflicts.  The exchange
// buffer Y holds a frame's n1 rows of n2 complex values (row k1 written by
// the first pass, read whole by one second-pass thread).  A frame's second-
// pass threads read their rows in step, so rows of an even length would put
// them on the same banks (n2 = 32: 64 floats apart, 16 threads on one bank);
// even rows are therefore padded to n2 + 1 complex values.  Frames follow at
// a stride of n1 * row + kExchangePad (a pad of 4 complex values spreads the
// frames of a wave over the 64 banks).  The power tile P holds each frame's
// n_fft/2 + 1 bins at a stride of n_fft/2 + 1 + kPowerPad (odd: no pad).
constexpr int kExchangePad = 4;
constexpr int kPowerPad = 0;
constexpr int exchange_row(int n2) { return n2 % 2 == 0 ? n2 + 1 : n2; }
constexpr int exchange_stride(int n1, int n2) { return n1 * exchange_row(n2) + kExchangePad; }
// The backward's exchange buffer (its second pass walks single rows).
constexpr int kBwdExchangePad = 4;
constexpr int bwd_exchange_stride(int half) { return half + kBwdExchangePad; }
constexpr int power_stride(int half) { return half + 1 + kPowerPad; }

// Backward pass: the filters that touch one one-sided bin.  A triangular
// filterbank puts every bin in at most two filters; an unused tap has
// m = n_mels (a zero row of the kernel's gradient tile) and weight 0.
struct BinTap {
  int32_t m0, m1;
  float w0, w1;
};

// Threads of a backward workgroup: 256 for every shape.  (n_fft = 2048
// tiles fill a CU's LDS on their own; at 256 threads a wave may use 512
// registers, which the two 32-point rows of its second pass need.)
constexpr int kBwdThreads = 256;
constexpr int kBwdLdsMax = 160 * 1024;  // LDS of a CU
// Waves per SIMD the backward kernel is built for: 2 (<= 256 registers each)
// up to n_fft = 1024, else 1.
constexpr int bwd_min_waves(int n1, int n2) { return n1 * n2 <= 512 ? 2 : 1; }

// Most frames one backward pass of a workgroup can hold: its second FFT
// pass gives each thread one frame's row (n1 <= 8: threads / n1 frames) or
// pair of rows (threads / (n1/2) frames), and shapes with n1 <= 8 keep every
// frame's samples of a pass in registers (at most 4 rounds of threads / n2
// frames).
constexpr int bwd_chunk_cap(int n1, int n2, int threads) {
  const int pass2 = n1 <= 8 ? threads / n1 : threads / (n1 / 2);
  const int pass1 = n1 <= 8 ? 4 * (threads / n2) : 64;
  const int c = pass2 < pass1 ? pass2 : pass1;
  return c < 64 ? c : 64;
}

// Forward kernel variants.
constexpr int kFwdSplit = 0;
constexpr int kFwdPaired = 1;
constexpr int kFwdLarge = 2;
constexpr int kFwdRows = 3;
constexpr int kFwdAuto = 4;  // ROWS or SPLIT, chosen per call (choose_forward)
// Row layout of the split kernel (fm_kernel.h, ROWS): threads per workgroup
// (one second-pass thread per row: N1 per frame, 64 frames at N1 = 8), and
// waves per SIMD it is built for: four (two tiles per CU, <= 128 registers)
// where its rows are short and its pass 1 keeps samples in registers, else two.
constexpr int kRowsThreads = 512;
constexpr int kRowsMaxN1 = 32;  // built for n1 <= 32 (fm_kernel.h kRowsCapable)
constexpr int rows_waves_per_simd(int n1, int n2) { return (n1 <= 16 && n2 <= 25) ? 4 : 2; }
// Shapes with a whole-tile sample copy (fm_kernel.h's COPY variant, chosen
// per call): those whose pass-1 threads hold all their samples in registers
// (n1 <= 8) and load two or more frames each, and those with larger n1,
// whose copy serves tiles of at most one frame per pass-1 thread.
constexpr bool copy_capable(int n1, int n2) { return n1 > 8 || n2 >= 8; }
// Paired kernel: R x R complex points per frame pair (n_fft = R*R); shapes
// built into the library.
constexpr int pair_radix_for(int n_fft) { return n_fft == 400 ? 20 : 0; }
constexpr int kPairThreadsHost = 256;
constexpr int kPairSpanFloatsHost = 4096;
constexpr int kPairOutPitchHost = 36;
// Layout of the paired kernel's LDS for radix r, chunks of `chunk` frames,
// n_mels filters and `w_floats` mel weights; returns the total bytes (offsets
// through the pointers: span buffer bytes, weights floats).
int pair_lds_layout(int r, int chunk, int n_mels, long w_floats, int* span_b, int* w_f);

// Threads per workgroup of an FFT shape.  n_fft = 2048 (32 x 32) tiles fill
// the LDS of a CU on their own; 8 waves instead of 4 give the CU two waves
// per SIMD and each pass-1 thread a single frame.
constexpr int threads_for(int n1, int n2) { return (n1 == 32 && n2 == 32) ? 512 : 256; }

// FFT factorisation of the complex transform of n_fft/2 points that carries
// the real FFT (even samples as real part, odd samples as imaginary part).
struct FftShape {
  int n1, n2;  // n_fft/2 = n1 * n2
  int n3 = 0;  // three-pass shapes (the large-FFT kernel): n_fft/2 = n1 * n2 * n3
};

// Large-FFT kernel (fm_large.h): n_fft/2 = a * c * d complex points in three
// register passes over one LDS buffer, c * d threads, one frame at a time.
// LDS strides in complex values: d + 1 per c, an odd c (d + 1) + 1 per a;
// the CSR mel weights (nnz floats, in 16-byte pieces) follow the buffer.
constexpr int large_threads(int c, int d) { return c * d; }
constexpr int large_exchange_bytes(int a, int c, int d) { return a * (c * (d + 1) + 1) * 8; }
constexpr int large_lds_bytes(int a, int c, int d, int nnz) {
  return large_exchange_bytes(a, c, d) + (nnz + 3) / 4 * 16;
}
// Frames one large-kernel workgroup takes at most per launch.
constexpr int kLargeTileMax = 1024;
// Three-pass shape that may serve the forward calls of a two-pass size
// (n_fft 4096: 2048 = 16 * 16 * 8), or n3 == 0.
constexpr FftShape large_alt_shape_for(int n_fft) {
  return n_fft == 4096 ? FftShape{16, 16, 8} : FftShape{0, 0, 0};
}

struct Plan {
  // transform arguments
  int sample_rate = 0, n_fft = 0, win_length = 0, hop = 0, n_mels = 0;
  double f_min = 0, f_max = 0, power = 2.0;
  int center = 1, pad_mode = FM_PAD_REFLECT, mel_scale = FM_MEL_HTK, norm = FM_NORM_NONE;
  int zpad = 0;                          // zero samples added on both sides
  int normalized = FM_NORMALIZED_NONE;
  int out_dtype = FM_F32;
  // derived
  int n_freqs = 0;     // n_fft/2 + 1
  int pad_left = 0;    // samples of centre padding on each side
  FftShape fft{0, 0};
  int tile_max = 0;      // most frames a workgroup tile may hold
  int tile_override = 0; // FM_TILE_FRAMES, for sweeps (0: chosen per call)
  int copy_override = -1; // FM_TILE_COPY=0|1, for A/B measurements (-1: chosen per call)
  int prio_override = -1; // FM_PRIO=0|1, for A/B measurements (-1: chosen per call)
  int threads = 256;
  int lds_bytes = 0;     // dynamic LDS of a tile of tile_max frames
  // mel blocks in wave order: wave w takes blocks [wave_beg[w], wave_beg[w+1])
  std::vector<MelBlock> blocks;
  int wave_beg[kMelWaves + 1] = {};
  std::vector<float> blk_w;            // block weights (see MelBlock)
  bool w_in_lds = true;                // weights staged in LDS (else read from L2)
  // vector-unit projection of wide tiles (kMelValuMinFrames): quads of 4
  // filters; quad q's header at quad_hdr[kQuadHdr*q], its weights at
  // quad_w[4 * (header offset) ...], 4 per step
  std::vector<int32_t> quad_hdr;
  std::vector<float> quad_w;
  int quad_beg[kMelShares + 1] = {};  // share s: quads [quad_beg[s], quad_beg[s+1])
  int mel_valu = 1;                   // 0 (FM_MEL=mfma): every tile projects on the matrix cores
  int mel_valu_from = kMelValuMinFrames;  // tiles of at least this many frames use the vector units
  int nnz = 0, w_max = 0;
  // host tables (float32 after one rounding from float64)
  std::vector<float> window;  // [n_fft], unscaled
  std::vector<MelRow> rows;   // [n_mels]
  std::vector<float> mel_w;   // [nnz]
  std::vector<float> tw_m;    // [2*M] exp(-2 pi i j / M), M = n_fft/2
  std::vector<float> tw_p;    // [2*M] first-pass twiddles in the order the pass reads
                              // them: entry k1*n2 + j = tw_m entry (j*k1) mod M
                              // (two-pass shapes; zero for the three-pass ones)
  std::vector<float> tw_n;    // [2*M] exp(-2 pi i k / n_fft)
  // device
  bool has_device = false;
  int device = -1;
  int n_cu = 0;                // compute units of that device
  std::vector<int> wg_per_cu;  // [tile frames] resident workgroups per CU
  void* d_block = nullptr;     // one allocation holding every table
  const void* d_win2 = nullptr;   // float2[M] : 0.5*(w[2m], w[2m+1])
  const void* d_tw_p = nullptr;   // float2[M] (right behind d_win2)
  const void* d_tw_m = nullptr;   // float2[M]
  const void* d_tw_n = nullptr;   // float2[M]
  const void* d_rows = nullptr;   // MelRow[n_mels]
  const void* d_mel_w = nullptr;  // float[nnz]
  const void* d_mel_tbl = nullptr;    // int32[8 + 4*n_blocks]: wave_beg, pad, blocks
  const void* d_blk_w = nullptr;      // float[blk_w.size()]
  const void* d_quad = nullptr;       // int32[16 + kQuadHdr*quads]: quad_beg, pad, headers
  const void* d_quad_w = nullptr;     // float[quad_w.size()]
  // forward kernel variant: FM_FWD_SPLIT (fm_kernel.h: complex FFT of n_fft/2
  // points and the real split, one tile per workgroup), FM_FWD_ROWS
  // (fm_kernel.h with one second-pass thread per row), FM_FWD_AUTO
  // (one of those two per call), FM_FWD_PAIRED (fm_pair.h: two frames per
  // complex FFT of n_fft points) or FM_FWD_LARGE (fm_large.h: n_fft 8192 and
  // 16384, three FFT passes, one frame at a time)
  int fwd_variant = 0;
  std::vector<int> rows_wg_per_cu;  // [tile frames] resident row-kernel workgroups per CU
  int pair_r = 0;              // paired: n_fft = pair_r * pair_r
  int pair_chunk = 0;          // paired: frames per chunk at most (even)
  int pair_lds_bytes = 0;      // paired: dynamic LDS per workgroup
  int pair_span_lds = 0;       //   byte offset of the sample span buffer
  int pair_w_lds = 0;          //   float offset of the mel weights
  int pair_wg_per_cu = 1;      // paired: resident workgroups per CU (device)
  int large_wg_per_cu = 1;     // large-FFT kernel: resident workgroups per CU (device)
  // The three-pass kernel serving forward calls: the plan's own shape for
  // n_fft 8192 and 16384; for n_fft 4096 a second kernel beside the split
  // one (fft 64 x 32, which also backs the backward), chosen per call.
  FftShape lfft{0, 0, 0};      // n3 == 0: none
  int large_threads = 0;       // its workgroup size (n2 * n3)
  int large_lds = 0;           // its dynamic LDS per workgroup
  int large_override = -1;     // FM_FORWARD=large|split at n_fft 4096, for A/B (-1: per call)
  // backward
  std::vector<BinTap> taps;      // [n_fft/2 + 1]
  int bwd_chunk_max = 0;         // frames per backward pass at most
  int bwd_chunk_override = 0;    // FM_BWD_CHUNK, for sweeps (0: chosen per call)
  std::vector<int> bwd_wg_per_cu;  // [chunk frames] resident backward workgroups per CU
  const void* d_taps = nullptr;  // BinTap[n_fft/2 + 1]
};

// Thread-local error reporting.
int set_error(int code, const std::string& msg);
const char* last_error_cstr();

// Builds every host table and the tile geometry; touches no GPU.
int build_host_plan(Plan& p, const fm_args& a);
void default_args(fm_args* a);

// LDS layout of a tile of `frames` frames: the FFT exchange buffer (during
// pass 1 followed by the pass-1 tables where tables_in_lds), which later
// holds the power tile, its zeroed overrun floats, (from float
// tile_weights_offset) the mel block weights and, for wide tiles, the mel
// waves' output staging areas right after them (mel_stage_floats: `rows` is
// the second pass's layout); behind all of that (byte tile_twiddles_offset),
// where twiddles_in_lds, the split twiddles W_N^k, k < n_fft/2.
int tile_exchange_bytes(const Plan& p, int frames);
int tile_weights_offset(const Plan& p, int frames);
int tile_tables_offset(const Plan& p, int frames);  // bytes; pass-1 tables in LDS
// Split twiddles W_N^k copied into LDS (complex FFTs of 1024 points or more;
// smaller ones hold them in registers or read them from L2).
constexpr bool twiddles_in_lds(int m) { return m >= 1024; }
int tile_twiddles_offset(const Plan& p, int frames, bool rows);  // bytes; split twiddles in LDS
// Tiles of this many frames project on the vector units (no block weights
// or staging in their LDS).
bool tile_mel_valu(const Plan& p, int frames);
int tile_lds_bytes(const Plan& p, int frames, bool rows);

// LDS layout of a backward pass of `chunk` frames (floats from the start):
// the exchange buffer (frame stride n_fft/2 + 4 complex), which after the
// inverse transform holds the windowed frame gradients; at bwd_grad_offset
// the bin gradients dP[f][k] (frame stride n_fft/2 + 1, odd); at
// bwd_acc_offset the edge accumulators (2 * bwd_edge floats) and 2 floats
// per wave for block sums; at bwd_gtile_offset the output-gradient tile
// g[m][f] of the pass, n_mels + 1 rows (the last one zero).
int bwd_edge(const Plan& p);  // samples at each signal end owned by edge workgroups
int bwd_grad_offset(const Plan& p, int chunk);
int bwd_acc_offset(const Plan& p, int chunk);
int bwd_gtile_offset(const Plan& p, int chunk);  // output-gradient tile [n_mels][chunk]
int bwd_lds_bytes(const Plan& p, int chunk);

// Frames per signal for a plan (negative FM_E_* on invalid length).
int64_t out_frames(const Plan& p, int64_t length);

// Device side (fm_launch.hip).
int upload_plan(Plan& p);
void free_plan_device(Plan& p);
// (paired kernel entry points, fm_pair_*.hip)
template <int R>
void* pair_kernel_for(int in_dtype, int pmode);
// (large-FFT kernel entry points, fm_large_*.hip)
template <int A, int C, int D>
void* large_kernel_for(int in_dtype, int pmode);
// How a forward call of `batch` signals of T frames runs: kernel variant
// (never kFwdAuto), frames per tile (paired: per chunk), workgroups, and
// whether tiles copy their sample span into LDS first (COPY variant).
struct FwdChoice {
  int variant = kFwdSplit;
  int tile = 1;
  int64_t workgroups = 0;
  bool copy = false;
  bool phase_prio = false;  // waves raise their issue priority by phase (mel_forward_kernel)
};
FwdChoice choose_forward(const Plan& p, int64_t batch, int64_t T);
int launch_forward(const Plan& p, const void* in, int in_dtype, int64_t batch,
                   int64_t length, void* out, void* stream);
int launch_backward(const Plan& p, const float* in, int64_t batch, int64_t length,
                    const float* grad_out, float* grad_in, void* stream);

}  // namespace fm
