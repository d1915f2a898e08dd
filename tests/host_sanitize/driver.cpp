// Exercises the host half of the C ABI (plan building, table accessors,
// frame counts, argument validation) over a grid of configurations, for a
// build under AddressSanitizer and UndefinedBehaviorSanitizer: any invalid
// access or undefined operation aborts the run.  Test infrastructure.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "fm.h"

static int failures = 0;
#define EXPECT(c)                                                   \
  do {                                                              \
    if (!(c)) {                                                     \
      std::fprintf(stderr, "expectation failed: %s (line %d)\n", #c, __LINE__); \
      ++failures;                                                   \
    }                                                               \
  } while (0)

static void inspect(fm_plan* h) {
  fm_plan_info in;
  EXPECT(fm_plan_info_get(h, &in) == FM_OK);
  EXPECT(in.has_device == 0);
  std::vector<float> win(in.n_fft), w(in.nnz > 0 ? in.nnz : 1), twm(in.n_fft), twn(in.n_fft);
  std::vector<int32_t> first(in.n_mels), len(in.n_mels), off(in.n_mels);
  EXPECT(fm_plan_tables(h, win.data(), first.data(), len.data(), off.data(), w.data(), twm.data(),
                        twn.data()) == FM_OK);
  EXPECT(fm_plan_tables(h, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == FM_OK);
  int32_t nb = 0;
  int64_t nw = 0;
  EXPECT(fm_plan_mel_blocks(h, nullptr, nullptr, nullptr, &nb, &nw) == FM_OK);
  std::vector<int32_t> blocks(4 * (nb > 0 ? nb : 1)), wave_beg(5);
  std::vector<float> bw(nw > 0 ? nw : 1);
  EXPECT(fm_plan_mel_blocks(h, blocks.data(), wave_beg.data(), bw.data(), nullptr, nullptr) == FM_OK);
  int32_t nq = 0;
  int64_t nqw = 0;
  EXPECT(fm_plan_mel_quads(h, nullptr, nullptr, nullptr, &nq, &nqw) == FM_OK);
  EXPECT(nq == (in.n_mels + 3) / 4);
  std::vector<int32_t> qh(6 * (nq > 0 ? nq : 1)), qs(9);
  std::vector<float> qw(nqw > 0 ? nqw : 1);
  EXPECT(fm_plan_mel_quads(h, qh.data(), qs.data(), qw.data(), nullptr, nullptr) == FM_OK);
  EXPECT(qs[0] == 0 && qs[8] == nq);
  for (int q = 0; q < nq; ++q)
    for (int a = 0; a < 4; ++a) EXPECT(qh[6 * q + a] >= 0 && qh[6 * q + a] + qh[6 * q + 4] <= in.n_freqs);
  for (int m = 0; m < in.n_mels; ++m) {
    EXPECT(len[m] >= 0 && first[m] >= 0 && first[m] + len[m] <= in.n_freqs);
    EXPECT(off[m] >= 0 && off[m] + len[m] <= in.nnz);
  }
  for (int64_t L : {1LL, 2LL, 199LL, 200LL, 201LL, 4000LL, 480000LL, (1LL << 29), (1LL << 40)}) {
    const int64_t T = fm_out_frames(h, L);  // valid lengths give counts, invalid ones an error code
    for (int64_t batch : {0LL, 1LL, 8LL, 64LL}) {
      int v = -1, tile = -1;
      int64_t wg = -1;
      const int st = fm_forward_config(h, batch, L, &v, &tile, &wg);
      EXPECT((st == FM_OK) == (T > 0));
      if (st != FM_OK) continue;
      EXPECT(v == FM_FWD_SPLIT || v == FM_FWD_ROWS || v == FM_FWD_PAIRED || v == FM_FWD_LARGE);
      // n_fft 4096 (two-pass plan) may take the three-pass kernel per call
      EXPECT(v == in.forward_variant ||
             (in.forward_variant == FM_FWD_AUTO && v != FM_FWD_PAIRED && v != FM_FWD_LARGE) ||
             (in.n_fft == 4096 && in.forward_variant == FM_FWD_SPLIT && v == FM_FWD_LARGE));
      EXPECT(tile >= 1);
      if (v != FM_FWD_PAIRED) EXPECT(wg == batch * ((T + tile - 1) / tile));
    }
  }
  EXPECT(fm_forward_config(h, -1, 4000, nullptr, nullptr, nullptr) == FM_E_INVAL);
  // a host plan has no device tables: both passes refuse before touching memory
  EXPECT(fm_forward(h, nullptr, FM_F32, 1, 4000, nullptr, nullptr) == FM_E_NODEVICE);
  EXPECT(fm_backward(h, nullptr, 1, 4000, nullptr, nullptr, nullptr) == FM_E_NODEVICE);
}

int main() {
  const int n_ffts[] = {64, 128, 256, 400, 512, 1024, 2048, 4096, 8192, 16384};
  int made = 0, rejected = 0;
  for (int n_fft : n_ffts) {
    for (int wdiv : {1, 2}) {
      for (int hdiv : {1, 3, 4, 16}) {
        for (int n_mels : {1, 24, 80, 128, 256, 300}) {
          for (int mode = 0; mode < 4; ++mode) {
            for (int variant = 0; variant < 4; ++variant) {
              fm_args a;
              EXPECT(fm_args_default(&a) == FM_OK);
              a.sample_rate = variant == 3 ? 44100 : 16000;
              a.n_fft = n_fft;
              a.win_length = n_fft / wdiv - (wdiv == 2 ? 3 : 0);
              a.hop_length = n_fft / hdiv > 0 ? n_fft / hdiv : 1;
              a.n_mels = n_mels;
              a.f_min = variant == 1 ? 30.0 : 0.0;
              a.f_max = a.sample_rate / 2;
              a.power = variant == 2 ? 1.5 : (variant == 1 ? 1.0 : 2.0);
              a.center = variant == 2 ? 0 : 1;
              a.pad_mode = mode;
              a.mel_scale = variant == 1 ? FM_MEL_SLANEY : FM_MEL_HTK;
              a.norm = variant == 3 ? FM_NORM_SLANEY : FM_NORM_NONE;
              a.pad = variant == 1 ? 37 : 0;
              a.normalized = variant;  // 3: out of range, rejected
              a.out_dtype = variant == 2 ? FM_F16 : FM_F32;
              fm_plan* h = nullptr;
              const int st = fm_plan_create_args_host(&h, &a);
              if (st == FM_OK) {
                ++made;
                inspect(h);
                EXPECT(fm_plan_destroy(h) == FM_OK);
              } else {
                ++rejected;
                EXPECT(h == nullptr);
                EXPECT(fm_strerror(st) != nullptr && fm_last_error() != nullptr);
              }
            }
          }
        }
      }
    }
  }
  // invalid arguments of every kind
  fm_args a;
  fm_args_default(&a);
  fm_plan* h = nullptr;
  fm_args b = a; b.n_fft = 300;           EXPECT(fm_plan_create_args_host(&h, &b) < 0);
  b = a; b.hop_length = 0;                EXPECT(fm_plan_create_args_host(&h, &b) < 0);
  b = a; b.win_length = 401;              EXPECT(fm_plan_create_args_host(&h, &b) < 0);
  b = a; b.f_min = 9000;                  EXPECT(fm_plan_create_args_host(&h, &b) < 0);
  b = a; b.f_max = 9000;                  EXPECT(fm_plan_create_args_host(&h, &b) < 0);
  b = a; b.power = -1;                    EXPECT(fm_plan_create_args_host(&h, &b) < 0);
  b = a; b.pad = -1;                      EXPECT(fm_plan_create_args_host(&h, &b) < 0);
  b = a; b.out_dtype = 7;                 EXPECT(fm_plan_create_args_host(&h, &b) < 0);
  b = a; b.sample_rate = 0;               EXPECT(fm_plan_create_args_host(&h, &b) < 0);
  EXPECT(fm_plan_create_args_host(nullptr, &a) == FM_E_INVAL);
  EXPECT(fm_plan_create_args_host(&h, nullptr) == FM_E_INVAL);
  EXPECT(fm_args_default(nullptr) == FM_E_INVAL);
  EXPECT(fm_plan_info_get(nullptr, nullptr) < 0);
  EXPECT(fm_out_frames(nullptr, 100) == FM_E_INVAL);
  EXPECT(fm_forward_config(nullptr, 1, 100, nullptr, nullptr, nullptr) == FM_E_INVAL);
  EXPECT(fm_plan_destroy(nullptr) == FM_OK);
  for (int s = -7; s <= 1; ++s) EXPECT(fm_strerror(s) != nullptr);
  std::printf("plans built %d, rejected %d, failures %d\n", made, rejected, failures);
  return failures == 0 && made > 1000 ? 0 : 1;
}
