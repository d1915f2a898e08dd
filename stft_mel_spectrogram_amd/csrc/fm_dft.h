// Register-resident small DFTs for the gfx950 kernel.
//
// Dft<R>::run(v) replaces v[0..R) (complex, natural order) by its DFT
// X[k] = sum_n v[n] exp(-2*pi*i*n*k/R), natural order.  Sizes are built from
// radix-2, -4 and -5 butterflies; a composite R = A*B runs A-point DFTs over
// the B decimated subsequences, multiplies by exp(-2*pi*i*b*ka/R) and runs
// B-point DFTs (mixed-radix Cooley-Tukey).  Every index and twiddle is a
// compile-time constant, so after unrolling the data stays in VGPRs and the
// twiddles are literal operands.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

namespace fm {

// ---- compile-time trigonometry on exact rationals --------------------------
constexpr double kTwoPi = 6.28318530717958647692528676655900577;

constexpr double sin_series(double x) {
  double x2 = x * x, t = x, s = x;
  for (int i = 1; i < 14; ++i) {
    t *= -x2 / static_cast<double>((2 * i) * (2 * i + 1));
    s += t;
  }
  return s;
}

constexpr double cos_series(double x) {
  double x2 = x * x, t = 1.0, s = 1.0;
  for (int i = 1; i < 14; ++i) {
    t *= -x2 / static_cast<double>((2 * i - 1) * (2 * i));
    s += t;
  }
  return s;
}

// cos(2*pi*j/n): the angle is folded into [0, pi/4] on integers first.
constexpr double cos_2pi(long j, long n) {
  long d = 8 * n;
  long a = ((j % n) + n) % n * 8;
  if (a > d / 2) a = d - a;
  double sign = 1.0;
  if (a > d / 4) {
    a = d / 2 - a;
    sign = -1.0;
  }
  if (a > d / 8) return sign * sin_series(kTwoPi * static_cast<double>(d / 4 - a) / static_cast<double>(d));
  return sign * cos_series(kTwoPi * static_cast<double>(a) / static_cast<double>(d));
}

// sin(2*pi*j/n) = cos(2*pi*(4j - n)/(4n))
constexpr double sin_2pi(long j, long n) { return cos_2pi(4 * j - n, 4 * n); }

// ---- compile-time loop -------------------------------------------------------
template <int I, int N, typename F>
__host__ __device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// ---- complex helpers on float2 -----------------------------------------------
__host__ __device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__host__ __device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__host__ __device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}

// v * exp(-2*pi*i*E/R) with E, R compile-time; the quarter turns are exact.
template <int E, int R>
__host__ __device__ __forceinline__ float2 twiddle(float2 v) {
  constexpr int e = ((E % R) + R) % R;
  if constexpr (e == 0) {
    return v;
  } else if constexpr (4 * e == R) {
    return make_float2(v.y, -v.x);            // * (-i)
  } else if constexpr (2 * e == R) {
    return make_float2(-v.x, -v.y);           // * (-1)
  } else if constexpr (4 * e == 3 * R) {
    return make_float2(-v.y, v.x);            // * (+i)
  } else {
    constexpr float c = static_cast<float>(cos_2pi(e, R));
    constexpr float s = static_cast<float>(sin_2pi(e, R));
    // (x + iy)(c - is) = (xc + ys) + i(yc - xs)
    return make_float2(fmaf(v.x, c, v.y * s), fmaf(v.y, c, -(v.x * s)));
  }
}

// ---- DFT kernels -------------------------------------------------------------
template <int R>
struct Dft;

template <>
struct Dft<1> {
  __host__ __device__ __forceinline__ static void run(float2*) {}
};

template <>
struct Dft<2> {
  __host__ __device__ __forceinline__ static void run(float2* v) {
    float2 a = v[0], b = v[1];
    v[0] = cadd(a, b);
    v[1] = csub(a, b);
  }
};

template <>
struct Dft<4> {
  __host__ __device__ __forceinline__ static void run(float2* v) {
    float2 s02 = cadd(v[0], v[2]), d02 = csub(v[0], v[2]);
    float2 s13 = cadd(v[1], v[3]), d13 = csub(v[1], v[3]);
    v[0] = cadd(s02, s13);
    v[2] = csub(s02, s13);
    v[1] = make_float2(d02.x + d13.y, d02.y - d13.x);  // d02 - i*d13
    v[3] = make_float2(d02.x - d13.y, d02.y + d13.x);  // d02 + i*d13
  }
};

template <>
struct Dft<5> {
  __host__ __device__ __forceinline__ static void run(float2* v) {
    constexpr float c1 = static_cast<float>(cos_2pi(1, 5));
    constexpr float c2 = static_cast<float>(cos_2pi(2, 5));
    constexpr float s1 = static_cast<float>(sin_2pi(1, 5));
    constexpr float s2 = static_cast<float>(sin_2pi(2, 5));
    const float2 x0 = v[0];
    const float2 t1 = cadd(v[1], v[4]), t2 = cadd(v[2], v[3]);
    const float2 t3 = csub(v[1], v[4]), t4 = csub(v[2], v[3]);
    v[0] = cadd(x0, cadd(t1, t2));
    const float2 a1 = make_float2(fmaf(c1, t1.x, fmaf(c2, t2.x, x0.x)), fmaf(c1, t1.y, fmaf(c2, t2.y, x0.y)));
    const float2 a2 = make_float2(fmaf(c2, t1.x, fmaf(c1, t2.x, x0.x)), fmaf(c2, t1.y, fmaf(c1, t2.y, x0.y)));
    const float2 b1 = make_float2(fmaf(s1, t3.x, s2 * t4.x), fmaf(s1, t3.y, s2 * t4.y));
    const float2 b2 = make_float2(fmaf(s2, t3.x, -(s1 * t4.x)), fmaf(s2, t3.y, -(s1 * t4.y)));
    v[1] = make_float2(a1.x + b1.y, a1.y - b1.x);  // a1 - i*b1
    v[4] = make_float2(a1.x - b1.y, a1.y + b1.x);  // a1 + i*b1
    v[2] = make_float2(a2.x + b2.y, a2.y - b2.x);  // a2 - i*b2
    v[3] = make_float2(a2.x - b2.y, a2.y + b2.x);  // a2 + i*b2
  }
};

// R = A * B: input index n = B*a + b, output index k = ka + A*kb.
template <int R, int A>
struct DftComposite {
  static constexpr int B = R / A;
  static_assert(A * B == R, "bad factorisation");
  __host__ __device__ __forceinline__ static void run(float2* v) {
    float2 u[R];  // u[b*A + ka]
    static_for<0, B>([&](auto bi) {
      constexpr int b = decltype(bi)::value;
      float2 t[A];
      static_for<0, A>([&](auto ai) {
        constexpr int a = decltype(ai)::value;
        t[a] = v[B * a + b];
      });
      Dft<A>::run(t);
      static_for<0, A>([&](auto ki) {
        constexpr int ka = decltype(ki)::value;
        u[b * A + ka] = twiddle<b * ka, R>(t[ka]);
      });
    });
    static_for<0, A>([&](auto ki) {
      constexpr int ka = decltype(ki)::value;
      float2 s[B];
      static_for<0, B>([&](auto bi) {
        constexpr int b = decltype(bi)::value;
        s[b] = u[b * A + ka];
      });
      Dft<B>::run(s);
      static_for<0, B>([&](auto kbi) {
        constexpr int kb = decltype(kbi)::value;
        v[ka + A * kb] = s[kb];
      });
    });
  }
};

// R = A * B with gcd(A, B) = 1 (Good-Thomas prime-factor algorithm): the
// input index n = (B*a + A*b) mod R and the output index k with k = ka
// (mod A), k = kb (mod B) turn the DFT into A-point DFTs over a followed by
// B-point DFTs over b with no twiddle factors between them, because
// exp(-2 pi i n k / R) = exp(-2 pi i a ka / A) * exp(-2 pi i b kb / B).
constexpr int mod_inverse(int x, int m) {
  for (int y = 1; y < m; ++y)
    if ((x * y) % m == 1) return y;
  return 0;
}
template <int R, int A>
struct DftPrimeFactor {
  static constexpr int B = R / A;
  static_assert(A * B == R && mod_inverse(B % A, A) > 0, "factors must be coprime");
  static constexpr int CA = B * mod_inverse(B % A, A);  // 1 mod A, 0 mod B
  static constexpr int CB = A * mod_inverse(A % B, B);  // 0 mod A, 1 mod B
  __host__ __device__ __forceinline__ static void run(float2* v) {
    float2 u[R];  // u[b*A + ka]
    static_for<0, B>([&](auto bi) {
      constexpr int b = decltype(bi)::value;
      float2 t[A];
      static_for<0, A>([&](auto ai) {
        constexpr int a = decltype(ai)::value;
        t[a] = v[(B * a + A * b) % R];
      });
      Dft<A>::run(t);
      static_for<0, A>([&](auto ki) {
        constexpr int ka = decltype(ki)::value;
        u[b * A + ka] = t[ka];
      });
    });
    static_for<0, A>([&](auto ki) {
      constexpr int ka = decltype(ki)::value;
      float2 s[B];
      static_for<0, B>([&](auto bi) {
        constexpr int b = decltype(bi)::value;
        s[b] = u[b * A + ka];
      });
      Dft<B>::run(s);
      static_for<0, B>([&](auto kbi) {
        constexpr int kb = decltype(kbi)::value;
        v[(ka * CA + kb * CB) % R] = s[kb];
      });
    });
  }
};

template <> struct Dft<8> : DftComposite<8, 2> {};
template <> struct Dft<10> : DftPrimeFactor<10, 2> {};
template <> struct Dft<20> : DftPrimeFactor<20, 4> {};
template <> struct Dft<16> : DftComposite<16, 4> {};
template <> struct Dft<25> : DftComposite<25, 5> {};
template <> struct Dft<32> : DftComposite<32, 4> {};
template <> struct Dft<64> : DftComposite<64, 8> {};

}  // namespace fm
