// Host plan builder for the fused mel-spectrogram forward pass.
//
// Everything the kernel reads besides the signal is built here once per plan,
// in float64, and rounded once to float32:
//   * the STFT window: periodic Hann of win_length, zero-padded centred to
//     n_fft, with the window / frame-length normalisation folded in
//     (flashmel 0.1.0 page, flashmel/filters.py make_window);
//   * the triangular mel filterbank in CSR form -- per mel the first bin of
//     its contiguous support, the run length and the weights -- with empty
//     filters kept as zero-length rows (flashmel/filters.py pack_fbank keeps
//     per-mel start/width rows; README "How it works": the projection loop
//     runs over each filter's actual width);
//   * from the CSR rows, the blocks the kernel's matrix-core projection
//     uses: 16 filters each over their common run of bins, dense in 4-bin
//     steps in the MFMA operand order, shared out over the waves;
//   * the twiddle tables of the complex FFT of n_fft/2 points that carries
//     the real FFT, and of the real-FFT post-processing step;
//   * the tile geometry of the kernel launch.
// No GPU is touched here, so CPU tests can inspect every table.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <sstream>

#include "fm_internal.h"

namespace fm {

namespace {

constexpr double kPi = 3.14159265358979323846264338327950288;

// cos and sin of 2*pi*j/n with the angle folded into [0, pi/4] in exact
// integer arithmetic before any rounding, so table entries are within one
// float64 rounding of the true values (before the final float32 rounding).
void cos_sin_2pi(int64_t j, int64_t n, double* c, double* s) {
  int64_t d = 8 * n;                      // angle = 2*pi*a/d
  int64_t a = ((j % n) + n) % n * 8;      // a in [0, d)
  // Reduce to [0, d/8] tracking the octant symmetries.
  double sc = 1.0, ss = 1.0;
  if (a > d / 2) { a = d - a; ss = -1.0; }             // theta -> 2pi - theta
  if (a > d / 4) { a = d / 2 - a; sc = -sc; }          // theta -> pi - theta
  bool swap = false;
  if (a > d / 8) { a = d / 4 - a; swap = true; }       // theta -> pi/2 - theta
  double th = 2.0 * kPi * static_cast<double>(a) / static_cast<double>(d);
  double cr = std::cos(th), sr = std::sin(th);
  if (swap) std::swap(cr, sr);
  *c = sc * cr;
  *s = ss * sr;
}

double hz_to_mel(double f, int scale) {
  if (scale == FM_MEL_HTK) return 2595.0 * std::log10(1.0 + f / 700.0);
  // Slaney: linear below 1 kHz (200/3 Hz per mel), log above (27 mel per x6.4)
  const double f_sp = 200.0 / 3.0, min_log_hz = 1000.0;
  const double min_log_mel = min_log_hz / f_sp, logstep = std::log(6.4) / 27.0;
  if (f >= min_log_hz) return min_log_mel + std::log(f / min_log_hz) / logstep;
  return f / f_sp;
}

double mel_to_hz(double m, int scale) {
  if (scale == FM_MEL_HTK) return 700.0 * (std::pow(10.0, m / 2595.0) - 1.0);
  const double f_sp = 200.0 / 3.0, min_log_hz = 1000.0;
  const double min_log_mel = min_log_hz / f_sp, logstep = std::log(6.4) / 27.0;
  if (m >= min_log_mel) return min_log_hz * std::exp(logstep * (m - min_log_mel));
  return f_sp * m;
}

// Complex FFT of M = n_fft/2 points split as n1 * n2: the first pass runs
// n2 transforms of n1 points, the second n1 transforms of n2 points.
bool fft_shape_for(int n_fft, FftShape* s) {
  switch (n_fft) {
    case 64: *s = {8, 4}; return true;      // 32 = 8 * 4
    case 128: *s = {8, 8}; return true;     // 64 = 8 * 8
    case 256: *s = {8, 16}; return true;    // 128 = 8 * 16
    case 400: *s = {8, 25}; return true;    // 200 = 8 * 25 (radix 2*4, 5*5)
    case 512: *s = {16, 16}; return true;   // 256 = 16 * 16
    case 1024: *s = {32, 16}; return true;  // 512 = 32 * 16 (radix 4*8, 4*4)
    case 2048: *s = {32, 32}; return true;  // 1024 = 32 * 32
    case 4096: *s = {64, 32}; return true;  // 2048 = 64 * 32 (radix 8*8, 4*8)
    // three passes (the large-FFT kernel)
    case 8192: *s = {16, 16, 16}; return true;   // 4096 = 16 * 16 * 16
    case 16384: *s = {16, 16, 32}; return true;  // 8192 = 16 * 16 * 32
    default: return false;
  }
}

std::string fmt(const char* what, double v) {
  std::ostringstream o;
  o << what << " (got " << v << ")";
  return o.str();
}

}  // namespace

int tile_exchange_bytes(const Plan& p, int frames) {
  // complex exchange buffer Y[frames][exchange_stride]
  const long y = static_cast<long>(std::max(frames, 1)) * exchange_stride(p.fft.n1, p.fft.n2) * 8;
  return static_cast<int>((y + 15) / 16 * 16);
}

int tile_weights_offset(const Plan& p, int frames) {
  // after the power tile P[frames][power_stride] and its zeroed overrun,
  // 16-byte aligned
  const long f = static_cast<long>(std::max(frames, 1)) * power_stride(p.n_fft / 2) + kMelTileOverrun;
  return static_cast<int>((f + 3) / 4 * 4);
}

int tile_tables_offset(const Plan& p, int frames) { return tile_exchange_bytes(p, frames); }

bool tile_mel_valu(const Plan& p, int frames) { return p.mel_valu && frames >= p.mel_valu_from; }

int tile_twiddles_offset(const Plan& p, int frames, bool rows) {
  const long tables = tables_in_lds(p.fft.n1, p.n_fft / 2) ? 16L * (p.n_fft / 2) : 0;
  const long pass1 = tile_tables_offset(p, frames) + tables;
  // the matrix-core mel stage's weights and staging (none on the vector units)
  const bool valu = tile_mel_valu(p, frames);
  const long stage = valu ? 0 : mel_stage_floats(rows, frames);
  const long weights = (p.w_in_lds && !valu) ? static_cast<long>(p.blk_w.size()) : 0;
  const long after_fft = (static_cast<long>(tile_weights_offset(p, frames)) + weights + stage) * 4;
  return static_cast<int>((std::max<long>(pass1, after_fft) + 15) / 16 * 16);
}

int tile_lds_bytes(const Plan& p, int frames, bool rows) {
  const long twiddles = twiddles_in_lds(p.n_fft / 2) ? 8L * (p.n_fft / 2) : 0;
  return static_cast<int>(tile_twiddles_offset(p, frames, rows) + twiddles);
}

int pair_lds_layout(int r, int chunk, int n_mels, long w_floats, int* span_b, int* w_f) {
  const int nf = r * r;
  // exchange buffer (pairs x (n_fft + 4) complex), which holds the tables at
  // the start and each chunk's output tile (n_mels rounded up to 16 rows of
  // kPairOutPitchHost floats) during the mel stage
  const long y = static_cast<long>(kPairThreadsHost / r) * (nf + 4) * 8;
  const long o = static_cast<long>((n_mels + 15) / 16 * 16) * kPairOutPitchHost * 4;
  const long region = (std::max(std::max(y, o), 8L * nf) + 15) / 16 * 16;
  // span buffer, later the power tile (chunk rows of n_fft/2 + 1 floats plus
  // the zeroed overrun)
  const long p_floats = static_cast<long>(chunk) * (nf / 2 + 1) + kMelTileOverrun;
  const long span = (std::max<long>(kPairSpanFloatsHost, p_floats) * 4 + 15) / 16 * 16;
  if (span_b) *span_b = static_cast<int>(region);
  if (w_f) *w_f = static_cast<int>((region + span) / 4);
  return static_cast<int>(region + span + 4 * w_floats);
}

int bwd_edge(const Plan& p) {
  // centre padding that copies signal samples hands gradients back to the
  // first and last n_fft/2 + 1 samples (constant padding copies none)
  return (p.center && p.pad_mode != FM_PAD_CONSTANT) ? p.pad_left + 1 : 0;
}

int bwd_grad_offset(const Plan& p, int chunk) {
  // after the exchange buffer Y[chunk][bwd_exchange_stride], 16-byte aligned
  const long y = static_cast<long>(std::max(chunk, 1)) * bwd_exchange_stride(p.n_fft / 2) * 8;
  return static_cast<int>((y + 15) / 16 * 4);
}

int bwd_acc_offset(const Plan& p, int chunk) {
  return bwd_grad_offset(p, chunk) + std::max(chunk, 1) * p.n_freqs;
}

int bwd_gtile_offset(const Plan& p, int chunk) {
  return bwd_acc_offset(p, chunk) + 2 * bwd_edge(p) + 2 * (kBwdThreads / 64);
}

int bwd_lds_bytes(const Plan& p, int chunk) {
  return (bwd_gtile_offset(p, chunk) + (p.n_mels + 1) * std::max(chunk, 1)) * 4;
}

int64_t out_frames(const Plan& p, int64_t length) {
  if (length < 1) return set_error(FM_E_INVAL, "length must be >= 1");
  const int64_t le = length + 2 * static_cast<int64_t>(p.zpad);  // zero-extended signal
  if (p.center) {
    if (p.pad_mode == FM_PAD_REFLECT && le <= p.pad_left)
      return set_error(FM_E_INVAL,
                       "reflect padding needs length + 2*pad > n_fft/2 (one reflection)");
    if (p.pad_mode == FM_PAD_CIRCULAR && le < p.pad_left)
      return set_error(FM_E_INVAL, "circular padding needs length + 2*pad >= n_fft/2 (one wrap)");
    int64_t lp = le + 2 * static_cast<int64_t>(p.pad_left);
    if (lp < p.n_fft) return set_error(FM_E_INVAL, "signal shorter than one frame");
    return 1 + (lp - p.n_fft) / p.hop;
  }
  if (le < p.n_fft) return set_error(FM_E_INVAL, "length + 2*pad < n_fft without centring");
  return 1 + (le - p.n_fft) / p.hop;
}

void default_args(fm_args* a) {
  *a = fm_args{};
  a->sample_rate = 16000;
  a->n_fft = 400;
  a->win_length = 400;
  a->hop_length = 200;
  a->n_mels = 128;
  a->f_min = 0.0;
  a->f_max = 8000.0;
  a->power = 2.0;
  a->center = 1;
  a->pad_mode = FM_PAD_REFLECT;
  a->mel_scale = FM_MEL_HTK;
  a->norm = FM_NORM_NONE;
  a->pad = 0;
  a->normalized = FM_NORMALIZED_NONE;
  a->out_dtype = FM_F32;
}

int build_host_plan(Plan& p, const fm_args& a) {
  const int sample_rate = a.sample_rate, n_fft = a.n_fft, win_length = a.win_length;
  const int hop_length = a.hop_length, n_mels = a.n_mels, center = a.center;
  const int pad_mode = a.pad_mode, mel_scale = a.mel_scale, norm = a.norm;
  const double f_min = a.f_min, f_max = a.f_max, power = a.power;
  // ---- validation (all host-side integer / float checks) ------------------
  if (sample_rate <= 0) return set_error(FM_E_INVAL, fmt("sample_rate must be > 0", sample_rate));
  if (n_fft <= 0) return set_error(FM_E_INVAL, fmt("n_fft must be > 0", n_fft));
  if (win_length <= 0 || win_length > n_fft)
    return set_error(FM_E_INVAL, fmt("need 0 < win_length <= n_fft", win_length));
  if (hop_length <= 0) return set_error(FM_E_INVAL, fmt("hop_length must be > 0", hop_length));
  if (n_mels <= 0) return set_error(FM_E_INVAL, fmt("n_mels must be > 0", n_mels));
  if (!(f_min >= 0.0) || !(f_max > f_min))
    return set_error(FM_E_INVAL, "need 0 <= f_min < f_max");
  if (f_max > sample_rate / 2.0)
    return set_error(FM_E_INVAL, fmt("f_max must be <= sample_rate/2", f_max));
  if (!(power > 0.0) || !std::isfinite(power))
    return set_error(FM_E_INVAL, fmt("power must be a positive finite number", power));
  if (center != 0 && center != 1) return set_error(FM_E_INVAL, "center must be 0 or 1");
  if (pad_mode < FM_PAD_REFLECT || pad_mode > FM_PAD_CIRCULAR)
    return set_error(FM_E_INVAL, fmt("unknown pad_mode", pad_mode));
  if (mel_scale != FM_MEL_HTK && mel_scale != FM_MEL_SLANEY)
    return set_error(FM_E_INVAL, fmt("unknown mel_scale", mel_scale));
  if (norm != FM_NORM_NONE && norm != FM_NORM_SLANEY)
    return set_error(FM_E_INVAL, fmt("unknown norm", norm));
  if (a.pad < 0 || a.pad > (1 << 28)) return set_error(FM_E_INVAL, fmt("need 0 <= pad <= 2^28", a.pad));
  if (a.normalized < FM_NORMALIZED_NONE || a.normalized > FM_NORMALIZED_FRAME_LENGTH)
    return set_error(FM_E_INVAL, fmt("unknown normalized", a.normalized));
  if (a.out_dtype != FM_F32 && a.out_dtype != FM_F16)
    return set_error(FM_E_INVAL, fmt("out_dtype must be FM_F32 or FM_F16", a.out_dtype));
  if (n_mels > kMaxMels) return set_error(FM_E_UNSUPPORTED, fmt("n_mels > 256 is not supported", n_mels));
  FftShape fs;
  if (!fft_shape_for(n_fft, &fs))
    return set_error(FM_E_UNSUPPORTED, fmt("n_fft not built (supported: 400 and powers of two 64..16384)", n_fft));

  p.sample_rate = sample_rate; p.n_fft = n_fft; p.win_length = win_length;
  p.hop = hop_length; p.n_mels = n_mels; p.f_min = f_min; p.f_max = f_max;
  p.power = power; p.center = center; p.pad_mode = pad_mode;
  p.mel_scale = mel_scale; p.norm = norm;
  p.zpad = a.pad; p.normalized = a.normalized; p.out_dtype = a.out_dtype;
  p.n_freqs = n_fft / 2 + 1;
  p.pad_left = center ? n_fft / 2 : 0;
  p.fft = fs;
  p.threads = fs.n3 ? large_threads(fs.n2, fs.n3) : threads_for(fs.n1, fs.n2);
  const int M = n_fft / 2;

  // ---- window: periodic Hann of win_length, centred in n_fft, with the
  //      STFT normalisation folded in (flashmel/filters.py make_window) -----
  p.window.assign(n_fft, 0.0f);
  const int left = (n_fft - win_length) / 2;
  std::vector<double> wd(win_length);
  double sum_sq = 0.0;
  for (int n = 0; n < win_length; ++n) {
    double c, s;
    cos_sin_2pi(n, win_length, &c, &s);
    wd[n] = 0.5 - 0.5 * c;
    sum_sq += wd[n] * wd[n];
  }
  double wscale = 1.0;
  if (a.normalized == FM_NORMALIZED_WINDOW) wscale = 1.0 / std::sqrt(sum_sq);
  if (a.normalized == FM_NORMALIZED_FRAME_LENGTH) wscale = 1.0 / std::sqrt(static_cast<double>(win_length));
  for (int n = 0; n < win_length; ++n) p.window[left + n] = static_cast<float>(wd[n] * wscale);

  // ---- mel filterbank: triangles on the mel scale, CSR rows ---------------
  std::vector<double> fpts(n_mels + 2);
  const double m_lo = hz_to_mel(f_min, mel_scale), m_hi = hz_to_mel(f_max, mel_scale);
  for (int i = 0; i < n_mels + 2; ++i)
    fpts[i] = mel_to_hz(m_lo + i * (m_hi - m_lo) / (n_mels + 1), mel_scale);
  const double half_sr = static_cast<double>(sample_rate / 2);
  p.rows.assign(n_mels, MelRow{0, 0, 0, 0});
  p.mel_w.clear();
  p.w_max = 0;
  std::vector<double> wrow(p.n_freqs);
  for (int m = 0; m < n_mels; ++m) {
    const double lo = fpts[m], mid = fpts[m + 1], hi = fpts[m + 2];
    const double scale = (norm == FM_NORM_SLANEY) ? 2.0 / (hi - lo) : 1.0;
    int first = -1, last = -1;
    for (int k = 0; k < p.n_freqs; ++k) {
      const double f = static_cast<double>(k) * half_sr / static_cast<double>(p.n_freqs - 1);
      const double up = (f - lo) / (mid - lo);
      const double down = (hi - f) / (hi - mid);
      double w = std::min(up, down);
      w = w > 0.0 ? w * scale : 0.0;
      wrow[k] = w;
      if (w > 0.0) {
        if (first < 0) first = k;
        last = k;
      }
    }
    MelRow r{0, 0, static_cast<int32_t>(p.mel_w.size()), 0};
    if (first >= 0) {
      r.first = first;
      r.len = last - first + 1;
      for (int k = first; k <= last; ++k) p.mel_w.push_back(static_cast<float>(wrow[k]));
      p.w_max = std::max(p.w_max, r.len);
    }
    p.rows[m] = r;
  }
  p.nnz = static_cast<int>(p.mel_w.size());

  // ---- backward taps: the (at most two) filters of every bin -------------
  // A bin at frequency f has a positive weight in filter m only when
  // f_pts[m] < f < f_pts[m+2]; with increasing corners that holds for two
  // consecutive filters at most.
  p.taps.assign(p.n_freqs, BinTap{n_mels, n_mels, 0.0f, 0.0f});
  {
    std::vector<int> used(p.n_freqs, 0);
    for (int m = 0; m < n_mels; ++m)
      for (int j = 0; j < p.rows[m].len; ++j) {
        const int k = p.rows[m].first + j;
        const float w = p.mel_w[p.rows[m].off + j];
        if (used[k] == 0) {
          p.taps[k].m0 = m;
          p.taps[k].w0 = w;
        } else if (used[k] == 1) {
          p.taps[k].m1 = m;
          p.taps[k].w1 = w;
        } else {
          return set_error(FM_E_UNSUPPORTED, "a frequency bin lies in more than two mel filters");
        }
        ++used[k];
      }
  }

  // ---- twiddles ------------------------------------------------------------
  p.tw_m.assign(2 * M, 0.0f);
  p.tw_n.assign(2 * M, 0.0f);
  for (int j = 0; j < M; ++j) {
    double c, s;
    cos_sin_2pi(j, M, &c, &s);
    p.tw_m[2 * j] = static_cast<float>(c);
    p.tw_m[2 * j + 1] = static_cast<float>(-s);
    cos_sin_2pi(j, n_fft, &c, &s);
    p.tw_n[2 * j] = static_cast<float>(c);
    p.tw_n[2 * j + 1] = static_cast<float>(-s);
  }
  // the first pass's twiddles exp(-2 pi i n2 k1 / M) in [k1][n2] order, so
  // that the threads of a pass (consecutive n2) read consecutive entries
  p.tw_p.assign(2 * M, 0.0f);
  if (fs.n3 == 0) {
    for (int k1 = 0; k1 < fs.n1; ++k1)
      for (int n2 = 0; n2 < fs.n2; ++n2) {
        const int e = (n2 * k1) % M;
        p.tw_p[2 * (k1 * fs.n2 + n2)] = p.tw_m[2 * e];
        p.tw_p[2 * (k1 * fs.n2 + n2) + 1] = p.tw_m[2 * e + 1];
      }
  }

  // ---- mel blocks ----------------------------------------------------------
  // Blocks of up to 16 filters; each covers the union of its filters' bin runs,
  // rounded up to whole groups of 4-bin steps and shifted left if it would
  // run past the last bin.  When 4*steps exceeds n_freqs it starts at bin 0
  // and reads at most 15 floats past a frame's row, all with zero weights:
  // the next frame's first bins, or, after the last valid frame of a tile
  // (full or ragged), floats the kernel zeroes before the mel stage.
  {
    const int K = p.n_freqs;
    auto make_block = [&](int m0, int m1, std::vector<float>& w) {
      int lo = K, hi = 0;
      for (int m = m0; m < m1; ++m)
        if (p.rows[m].len > 0) {
          lo = std::min(lo, static_cast<int>(p.rows[m].first));
          hi = std::max(hi, static_cast<int>(p.rows[m].first + p.rows[m].len));
        }
      MelBlock b{0, 0, 0, m0};
      b.nrow = m1 - m0;
      w.clear();
      if (hi > lo) {
        b.ksteps = ((hi - lo + 3) / 4 + kMelStepGroup - 1) / kMelStepGroup * kMelStepGroup;
        b.kb = std::max(0, std::min(lo, K - 4 * b.ksteps));
        w.assign(static_cast<size_t>(b.ksteps) * 64, 0.0f);
        for (int s = 0; s < b.ksteps; ++s)
          for (int l = 0; l < 64; ++l) {
            const int m = m0 + l % kMelBlock, k = b.kb + 4 * s + l / kMelBlock;
            if (m >= m1) continue;
            const MelRow& r = p.rows[m];
            if (r.len > 0 && k >= r.first && k < r.first + r.len) {
              w[static_cast<size_t>(s) * 64 + l] = p.mel_w[r.off + k - r.first];
              b.s_hi = std::max(b.s_hi, s + 1);
            }
          }
      }
      return b;
    };
    // 16 consecutive filters per block; then, while the longest block runs
    // more than 32 steps and more than twice an eighth of all steps (the mel
    // stage spreads over up to 8 waves, and each block is one wave's serial
    // chain of steps), it is split into its two halves of filters, each over
    // its own (shorter) bin run.  A filter's sum is the same either way: its
    // bins all lie in its block's run, and the steps go in bin order.
    // Measured (same box, us per launch, narrow tiles on the matrix cores):
    // n_fft 1024, 8 x 32768 (longest block 60 -> 36 steps): 8.31 -> 8.00;
    // n_fft 2048, 64 x 220500 (88 -> 60): 83.3 -> 81.5; n_fft 4096, 4 x
    // 1323000: 60.5 -> 58.1.  Splitting shorter blocks, or down to 5/4 of an
    // eighth, adds more steps than it saves (n_fft 400, 1 x 16000: 6.52 ->
    // 6.67; n_fft 512, 32 x 480000: 56.0 -> 58.0).
    std::vector<std::pair<int, int>> ranges;
    for (int m0 = 0; m0 < n_mels; m0 += kMelBlock) ranges.push_back({m0, std::min(n_mels, m0 + kMelBlock)});
    std::vector<float> tmp, tmp2;
    for (int it = 0; it < 16; ++it) {
      long total = 0;
      int longest = -1, lsteps = 0;
      for (size_t r = 0; r < ranges.size(); ++r) {
        const int st = make_block(ranges[r].first, ranges[r].second, tmp).ksteps;
        total += st;
        if (st > lsteps) {
          lsteps = st;
          longest = static_cast<int>(r);
        }
      }
      if (longest < 0 || lsteps <= 32 || 4L * lsteps <= total) break;
      const int m0 = ranges[longest].first, m1 = ranges[longest].second;
      if (m1 - m0 < 2) break;
      const int mid = m0 + (m1 - m0) / 2;
      const int sa = make_block(m0, mid, tmp).ksteps, sb = make_block(mid, m1, tmp2).ksteps;
      if (std::max(sa, sb) >= lsteps) break;  // no shorter chain
      ranges[longest] = {m0, mid};
      ranges.insert(ranges.begin() + longest + 1, {mid, m1});
    }
    const int nb = static_cast<int>(ranges.size());
    std::vector<MelBlock> blk(nb);
    std::vector<std::vector<float>> bw(nb);
    for (int j = 0; j < nb; ++j) blk[j] = make_block(ranges[j].first, ranges[j].second, bw[j]);
    // Longest first onto the least loaded wave; a block costs its steps plus
    // 2 for the address set-up and the stores.
    std::vector<int> order(nb);
    for (int j = 0; j < nb; ++j) order[j] = j;
    std::stable_sort(order.begin(), order.end(),
                     [&](int x, int y) { return blk[x].ksteps > blk[y].ksteps; });
    long load[kMelWaves] = {};
    std::vector<int> owner(nb);
    for (int j : order) {
      int w = 0;
      for (int v = 1; v < kMelWaves; ++v)
        if (load[v] < load[w]) w = v;
      owner[j] = w;
      load[w] += blk[j].ksteps + 2;
    }
    // Within a share, longest first: where the row layout spreads a share over
    // two waves (alternate blocks), that balances them too.
    p.blocks.clear();
    p.blk_w.clear();
    for (int w = 0; w < kMelWaves; ++w) {
      p.wave_beg[w] = static_cast<int>(p.blocks.size());
      for (int j : order)
        if (owner[j] == w) {
          MelBlock b = blk[j];
          b.w_off = static_cast<int32_t>(p.blk_w.size());
          p.blk_w.insert(p.blk_w.end(), bw[j].begin(), bw[j].end());
          p.blocks.push_back(b);
        }
    }
    p.wave_beg[kMelWaves] = static_cast<int>(p.blocks.size());
    p.w_in_lds = M < kMelGlobalWeightsFrom;
    if (!p.w_in_lds)  // read-ahead slack of the chunked global loads
      p.blk_w.resize(p.blk_w.size() + static_cast<size_t>(kMelGlobalChunk) * 64, 0.0f);
    static_assert(kMelTileOverrun >= 4 * kMelStepGroup - 1, "zeroed tail too short");
    static_assert(kMelStepGroup * 64 % 256 == 0, "blocks must fill whole copy chunks");
  }
  // ---- filter quads (vector-unit projection of wide tiles) -----------------
  // Quad q holds filters 4q .. 4q+3, each over a run of L bins, L its
  // longest filter's run; a shorter run is padded with zero weights, and
  // starts early enough that the padded run ends inside the frame's bins.
  // Weights in step order, 4 per step (one per filter), so a step's four
  // weights are one 16-byte scalar load.
  {
    const int K = p.n_freqs;
    const int nq = (n_mels + 3) / 4;
    p.quad_hdr.assign(static_cast<size_t>(nq) * kQuadHdr, 0);
    p.quad_w.clear();
    std::vector<long> cost(nq);
    for (int q = 0; q < nq; ++q) {
      int L = 0;
      for (int a = 0; a < 4 && 4 * q + a < n_mels; ++a) L = std::max(L, static_cast<int>(p.rows[4 * q + a].len));
      int32_t* h = &p.quad_hdr[static_cast<size_t>(q) * kQuadHdr];
      h[4] = L;
      h[5] = static_cast<int32_t>(p.quad_w.size() / 4);
      p.quad_w.resize(p.quad_w.size() + 4 * static_cast<size_t>(L), 0.0f);
      float* w = p.quad_w.data() + 4 * static_cast<size_t>(h[5]);
      for (int a = 0; a < 4; ++a) {
        const int m = 4 * q + a;
        if (m >= n_mels || p.rows[m].len == 0) continue;  // start 0, zero weights
        const MelRow& r = p.rows[m];
        const int st = std::max(0, std::min(static_cast<int>(r.first), K - L));
        h[a] = st;
        for (int i = 0; i < L; ++i) {
          const int k = st + i;
          if (k >= r.first && k < r.first + r.len) w[4 * i + a] = p.mel_w[r.off + k - r.first];
        }
      }
      cost[q] = L + 3;  // the steps, plus the header loads and 4 row stores
    }
    // contiguous shares of about equal cost
    long total = 0;
    for (long c : cost) total += c;
    int q = 0;
    long acc = 0;
    p.quad_beg[0] = 0;
    for (int sh = 1; sh < kMelShares; ++sh) {
      const long target = (total * sh + kMelShares / 2) / kMelShares;
      while (q < nq && acc + cost[q] / 2 < target) acc += cost[q++];
      p.quad_beg[sh] = q;
    }
    p.quad_beg[kMelShares] = nq;
  }
  // the mel stage's implementation per tile width (tile_mel_valu), before the
  // tile geometry: it decides which tiles hold the block weights in LDS
  if (const char* e = std::getenv("FM_MEL")) {
    if (std::string(e) == "mfma") p.mel_valu = 0;
    if (std::string(e) == "valu") p.mel_valu = 1;
  }
  if (const char* e = std::getenv("FM_MEL_FROM")) {  // A/B of the threshold
    const int v = std::atoi(e);
    if (v >= 1 && v <= 64) p.mel_valu_from = v;
  }
  // ---- the three-pass kernel beside a two-pass size -------------------------
  // Chosen per call in choose_forward where its buffer plus the weights fit
  // the LDS.
  {
    const FftShape ls = large_alt_shape_for(n_fft);
    if (ls.n3 && large_lds_bytes(ls.n1, ls.n2, ls.n3, p.nnz) <= 160 * 1024) {
      p.lfft = ls;
      p.large_threads = large_threads(ls.n2, ls.n3);
      p.large_lds = large_lds_bytes(ls.n1, ls.n2, ls.n3, p.nnz);
      if (const char* e = std::getenv("FM_FORWARD")) {
        if (std::string(e) == "large") p.large_override = 1;
        if (std::string(e) == "split") p.large_override = 0;
      }
    }
  }
  // ---- tile geometry -------------------------------------------------------
  if (fs.n3) {
    // The large-FFT kernel holds one frame's exchange buffer and walks its
    // tile frame by frame; it has no backward kernel.
    p.tile_max = kLargeTileMax;
    p.lds_bytes = large_lds_bytes(fs.n1, fs.n2, fs.n3, p.nnz);
    if (p.lds_bytes > 160 * 1024)
      return set_error(FM_E_UNSUPPORTED, "mel filterbank too large for the LDS of one workgroup");
    p.bwd_chunk_max = 0;
    p.fwd_variant = kFwdLarge;
    p.lfft = fs;
    p.large_threads = p.threads;
    p.large_lds = p.lds_bytes;
    p.tile_override = 0;
    p.bwd_chunk_override = 0;
    if (const char* e = std::getenv("FM_TILE_FRAMES")) {
      int v = std::atoi(e);
      if (v >= 1 && v <= p.tile_max) p.tile_override = v;
    }
    return FM_OK;
  }
  // At most 64 frames per workgroup tile (four 16-frame column groups of
  // the mel stage's matrix products); the second FFT pass gives each thread
  // one pair of n2-point transforms; the tile's LDS (the exchange buffer, or
  // the power tile plus the mel weights) must fit the 160 KB of a CU.
  int tmax = 64;
  while (tmax > 1 && tmax * (fs.n1 / 2) > p.threads) --tmax;
  // (either layout of the second pass)
  // (either layout of the second pass; every width up to the maximum must fit:
  // tiles that project on the vector units hold no block weights, so a
  // narrower tile may need more LDS than a wider one)
  auto lds_of = [&](int g) { return std::max(tile_lds_bytes(p, g, false), tile_lds_bytes(p, g, true)); };
  auto lds_upto = [&](int g) {
    int m = 0;
    for (int h = 1; h <= g; ++h) m = std::max(m, lds_of(h));
    return m;
  };
  while (tmax > 1 && lds_upto(tmax) > 160 * 1024) --tmax;
  if (lds_upto(tmax) > 160 * 1024)
    return set_error(FM_E_UNSUPPORTED, "mel filterbank too large for the LDS of one tile");
  p.tile_max = tmax;
  p.lds_bytes = lds_upto(tmax);
  // backward passes: as many frames as the kernel's registers and the LDS
  // allow
  int cmax = bwd_chunk_cap(fs.n1, fs.n2, kBwdThreads);
  while (cmax > 1 && bwd_lds_bytes(p, cmax) > 160 * 1024) --cmax;
  p.bwd_chunk_max = bwd_lds_bytes(p, cmax) <= 160 * 1024 ? cmax : 0;
  // paired forward kernel where it is built and its chunks keep most of the
  // workgroup busy: two full passes of R threads per frame pair need
  // 2*floor(256/R) frames per chunk, whose samples ((chunk-1)*hop + n_fft,
  // plus alignment slack) fit the span buffer; FM_FORWARD=split|paired
  // overrides the choice (for A/B measurements)
  p.fwd_variant = kFwdSplit;
  p.pair_r = pair_radix_for(n_fft);
  if (p.pair_r > 0 && p.w_in_lds) {
    const int cmax = 2 * (kPairThreadsHost / p.pair_r);
    int c = cmax;
    while (c > 2 && static_cast<long>(c - 1) * hop_length + n_fft + 16 > kPairSpanFloatsHost) c -= 2;
    const bool fits = static_cast<long>(c - 1) * hop_length + n_fft + 16 <= kPairSpanFloatsHost;
    const int bytes = pair_lds_layout(p.pair_r, c, n_mels, static_cast<long>(p.blk_w.size()),
                                      &p.pair_span_lds, &p.pair_w_lds);
    p.pair_chunk = c;
    p.pair_lds_bytes = bytes;
    bool use = false;  // measured slower than the split kernel so far: opt-in only
    if (const char* e = std::getenv("FM_FORWARD")) {
      if (std::string(e) == "paired" && fits && bytes <= 160 * 1024) use = true;
    }
    if (use) p.fwd_variant = kFwdPaired;
  }
  // Row layout of the second pass (one thread per row of every frame of a
  // tile, so at most kRowsThreads / n1 frames): chosen per call
  // (choose_forward); FM_FORWARD=rows or split forces one layout (for A/B
  // measurements).
  if (p.fwd_variant == kFwdSplit && fs.n1 <= kRowsMaxN1 && tmax * fs.n1 <= kRowsThreads) {
    p.fwd_variant = kFwdAuto;
    if (const char* e = std::getenv("FM_FORWARD")) {
      if (std::string(e) == "rows") p.fwd_variant = kFwdRows;
      if (std::string(e) == "split") p.fwd_variant = kFwdSplit;
    }
  }
  p.tile_override = 0;
  p.bwd_chunk_override = 0;
  if (const char* e = std::getenv("FM_BWD_CHUNK")) {
    int v = std::atoi(e);
    if (v >= 1 && v <= p.bwd_chunk_max) p.bwd_chunk_override = v;
  }
  if (const char* e = std::getenv("FM_TILE_FRAMES")) {
    int v = std::atoi(e);
    if (v >= 1 && v <= tmax) p.tile_override = v;
  }
  if (const char* e = std::getenv("FM_TILE_COPY")) {
    if (std::string(e) == "0") p.copy_override = 0;
    if (std::string(e) == "1") p.copy_override = 1;
  }
  if (const char* e = std::getenv("FM_PRIO")) {
    if (std::string(e) == "0") p.prio_override = 0;
    if (std::string(e) == "1") p.prio_override = 1;
  }
  return FM_OK;
}

namespace {

// Resident workgroups per CU for a tile of g frames (1 where unknown: host
// plans, or sizes the device pass did not measure).
int occupancy(const std::vector<int>& tab, int g) {
  return (g < static_cast<int>(tab.size()) && tab[g] > 0) ? tab[g] : 1;
}

// Frames per tile for a tile-per-workgroup kernel of `threads` threads with
// residency table `occ`.  The busiest CU's workgroups, in rounds of up to k
// resident ones, where a round of j costs 1 + 0.7 (j - 1) workgroup times
// (they share the SIMDs), times the time of one workgroup, which grows with
// its pass-1 rounds (frames per thread) on top of a fixed part (pass 2,
// split, mel) worth about 3 of them; ties go to smaller tiles (more compute
// units busy for small calls).  Against counting whole rounds of k (same
// box, us per launch): n_fft 400, 4 x 480000: 47-frame tiles, one per CU,
// 9.89 against 32-frame ones 11.04; n_fft 512, 8 x 480000: 32 frames 17.12
// against 24 frames 18.12; n_fft 128, 8 / 16 x 480000: 16.62 / 31.79
// against 17.09 / 34.18; n_fft 64, 4 / 8 x 480000: 12.02 / 19.70 against
// 13.32 / 21.70; the other benchmark calls keep their tiles.  Earlier:
// n_fft 2048 x 64 signals picks 16 frames (7 rounds of 1 per CU: 127 us)
// where "fewest frames on the busiest CU" picked 12 (9 rounds: 160 us).  Calls with fewer tiles than CUs then shrink the
// tile while every tile still gets a CU of its own (1 x 16000 samples:
// 1-frame tiles, 8.2 us, against 10.0 us with 32-frame tiles; below that
// point, in calls of several rounds, the model above does not rank small
// tiles reliably and they measured slower).
int choose_tile(const Plan& p, int64_t batch, int64_t T, int threads, const std::vector<int>& occ) {
  if (p.tile_override > 0) return p.tile_override;
  const int64_t ncu = p.n_cu > 0 ? p.n_cu : 256;
  const int slots = std::max(1, threads / p.fft.n2);  // frames per pass-1 round
  int best = p.tile_max;
  int64_t best_cost = INT64_MAX;
  for (int g = (p.tile_max + 1) / 2; g <= p.tile_max; ++g) {
    const int64_t tiles = batch * ((T + g - 1) / g);
    const int64_t k = occupancy(occ, g);
    const int64_t w = (tiles + ncu - 1) / ncu;  // workgroups on the busiest CU
    // tenths of a workgroup's time per round of j resident workgroups: 10 +
    // 7 (j - 1) (they share the SIMDs)
    const int64_t span = (w / k) * (10 + 7 * (k - 1)) + (w % k ? 10 + 7 * (w % k - 1) : 0);
    const int64_t cost = span * ((g + slots - 1) / slots + 3);
    if (cost < best_cost) {
      best_cost = cost;
      best = g;
    }
  }
  // A call that leaves CUs idle takes smaller tiles, down to one per CU.
  if (batch * ((T + best - 1) / best) < ncu) {
    while (best > 1 && batch * ((T + best - 2) / (best - 1)) <= ncu) --best;
  }
  return best;
}

}  // namespace

// Kernel and tiling of one forward call.  FM_FWD_AUTO plans choose the
// second pass's layout per call, from same-box A/B measurements of the two
// (identical outputs):
// - n_fft 400 (8 x 25), 2048 (32 x 32), 256 (8 x 16) and 512 (16 x 16): rows
//   always.  At n_fft 2048 the
//   pair layout leaves half of its 512 threads idle in pass 2 at the
//   14-17-frame tiles that fit the LDS (64 x 220500: 94.1 against 103.1
//   us).  At n_fft 400 rows measured 1-17% faster at every call size tried
//   with the tile copy below (8 x 480000: 16.76-16.87 against 17.24-17.31
//   us; int16: 16.36 against 17.29; 16 x 480000: 30.3 against 32.5; 1 x
//   16000: 6.6 against 8.1).  At n_fft 256 and 512 (hop 64 and 160, with
//   the vector-unit mel stage) rows measured 1-9% faster at every call size
//   tried: n_fft 256, 2 / 4 / 8 / 16 x 480000: 8.22 / 10.13 / 18.43 / 34.79
//   against 8.56 / 10.56 / 20.33 / 36.96 us; n_fft 512: 8.36 / 9.87 / 18.14
//   / 28.97 against 8.51 / 10.17 / 18.19 / 30.54 us.
// - the other shapes built with both layouts: rows when its workgroups fit
//   one per compute unit (the latency-bound calls: n_fft 1024, 16 x 32768:
//   13.7 against 14.5 us); the pair layout for larger calls, where its
//   workgroups share the CUs with fewer barriers per frame (n_fft 1024,
//   32 x 32768: 17.3 against 24.1 us; n_fft 128, 8 x 480000: 17.4 against
//   22.4 us; n_fft 64: 21.8 against 23.5 us).
// Whole-tile sample copy (COPY variant; shapes with copy_capable): the
// exchange buffer (G x (n_fft/2 + 4) complex) holds a tile's span ((G-1)
// hop + n_fft samples + 32 bytes of alignment) whenever hop <= n_fft.  Every
// tile copies, the first and last of a signal too (their padding filled per
// sample), wherever frames overlap or touch (hop <= n_fft; with gaps between
// frames the span would carry samples no frame reads).  Against the
// per-frame gather (same box, us per launch): n_fft 400, 8 x 480000: 15.9
// against 16.6; int16: 14.7 against 16.5; 1 x 16000: 6.5 against 6.8; 1 x
// 480000: 7.5 against 7.9; n_fft 1024, 8 x 32768: 8.2 against 12.7; n_fft
// 2048, 8 x 220500: 13.9 against 17.5; 64 x 220500: 83.4 against 93.7;
// n_fft 512, 1 x 480000: 6.9 against 9.0; n_fft 4096, 1 x 1323000: 20.6
// against 34.7.  (While edge tiles gathered, the copy lost in calls of few
// workgroups: there the gathering edge tiles set the launch's length.)
FwdChoice choose_forward(const Plan& p, int64_t batch, int64_t T) {
  FwdChoice c;
  const int64_t ncu = p.n_cu > 0 ? p.n_cu : 256;
  const int64_t nb = std::max<int64_t>(batch, 1);
  if (p.fwd_variant == kFwdPaired) {
    c.variant = kFwdPaired;
    c.tile = p.pair_chunk;
    c.workgroups = std::min(batch * T, ncu * p.pair_wg_per_cu);
    return c;
  }
  // the three-pass kernel: the fewest frames per workgroup that put every
  // frame in the first round of resident workgroups (each walks its frames
  // one at a time)
  auto large = [&](int override_tile) {
    const int64_t slots = ncu * p.large_wg_per_cu;
    int64_t g = override_tile > 0 ? override_tile : 1;
    if (override_tile <= 0)
      while (g < kLargeTileMax && nb * ((T + g - 1) / g) > slots) ++g;
    FwdChoice l;
    l.variant = kFwdLarge;
    l.tile = static_cast<int>(g);
    l.workgroups = batch * ((T + g - 1) / g);
    return l;
  };
  if (p.fwd_variant == kFwdLarge) return large(p.tile_override);
  auto tile_copy = [&](int g) {
    if (!copy_capable(p.fft.n1, p.fft.n2)) return false;
    // the exchange buffer must hold the span ((g - 1) hop + n_fft samples of
    // up to 4 bytes, and up to 30 bytes of 16-byte rounding), also when forced
    if ((static_cast<long>(g - 1) * p.hop + p.n_fft) * 4 + 32 > tile_exchange_bytes(p, g)) return false;
    if (p.copy_override >= 0) return p.copy_override == 1;
    return p.hop <= p.n_fft;
  };
  c.variant = kFwdSplit;
  c.tile = choose_tile(p, nb, T, p.threads, p.wg_per_cu);
  c.workgroups = batch * ((T + c.tile - 1) / c.tile);
  c.copy = tile_copy(c.tile);
  // n_fft 4096: the three-pass kernel (16 x 16 x 8, two waves, several
  // resident per CU) once the split kernel's 8-frame tiles, one per CU at a
  // time, would take more than one round (same box, us per launch: 4 x
  // 1323000 samples 46.3 against 57.6; 16 x 1323000: 137.0 against 196.7;
  // 1 x 1323000, 216 tiles: 20.8 against 19.7)
  if (p.lfft.n3 && p.fwd_variant == kFwdSplit &&
      (p.large_override == 1 || (p.large_override < 0 && c.workgroups > ncu)))
    return large(p.large_override == 1 ? p.tile_override : 0);  // FM_TILE_FRAMES when forced
  if (p.fwd_variant != kFwdRows && p.fwd_variant != kFwdAuto) return c;
  const int rows_tile = choose_tile(p, nb, T, kRowsThreads, p.rows_wg_per_cu);
  const int64_t rows_tiles = nb * ((T + rows_tile - 1) / rows_tile);
  bool rows = p.fwd_variant == kFwdRows;
  if (p.fwd_variant == kFwdAuto) {
    const bool always = (p.fft.n1 == 32 && p.fft.n2 == 32) || (p.fft.n1 == 8 && p.fft.n2 == 25) ||
                        (p.fft.n1 == 8 && p.fft.n2 == 16) || (p.fft.n1 == 16 && p.fft.n2 == 16);
    rows = always || rows_tiles <= ncu;
  }
  if (rows) {
    c.variant = kFwdRows;
    c.tile = rows_tile;
    c.workgroups = batch * ((T + rows_tile - 1) / rows_tile);
    c.copy = tile_copy(rows_tile);
  }
  // Phase priorities: in a call of one round that puts two or more
  // workgroups on a CU, the older workgroup otherwise wins the SIMDs' issue
  // arbitration in every phase and its CU-mate, starved through pass 1,
  // finishes alone; with each wave's priority falling phase by phase (pass 1
  // highest, the mel stage lowest) the workgroup that is behind goes first.
  // Measured (same box, us per launch): n_fft 400, 8 x 480000: 14.35
  // against 14.98; int16 13.17 against 13.88; 4 x 480000: 11.61 against
  // 12.19.  In calls of several rounds it costs (16 x 480000: 29.0 against
  // 27.0), and with one workgroup per CU it has nothing to order (1 x 16000,
  // n_fft 1024 8 x 32768: within 1.2%).
  {
    const int occ = occupancy(c.variant == kFwdRows ? p.rows_wg_per_cu : p.wg_per_cu, c.tile);
    c.phase_prio = p.prio_override >= 0 ? p.prio_override == 1
                                        : (c.workgroups > ncu && c.workgroups <= ncu * occ);
  }
  return c;
}

}  // namespace fm
