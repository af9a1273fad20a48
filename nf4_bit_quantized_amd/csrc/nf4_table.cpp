// NF4 level table and nearest-level thresholds, built on the host.
//
// Levels ("QLoRA技术从入门到精通" §2(3); "【X 长文】LoRA 与 QLoRA：用一块 GPU
// 微调大模型", NF4 paragraph): normal quantiles placed as the medians of
// equal-probability slices, dense near 0, with an exact 0, 16 levels in
// [-1, 1].  With 16 equal slices of the whole normal there is no zero level,
// so the table is built as 7 equal slices of the lower half and 8 of the
// upper half, each slice represented by its median, each half scaled by its
// largest magnitude (ends exactly -1 and +1), plus the level 0; ascending.
//
// The inverse normal CDF is computed here by Newton iteration on the
// complementary error function of the C library, in double precision, and
// the levels are rounded to float32 once.
//
// The uniform table ("7、QLoRA 量化微调" §7.1): 16 equally spaced levels
// -1 + 2i/15 on [-1, 1] (computed in double, rounded to float32 once); it has
// no zero level.  Same thresholds rule.
//
// Thresholds: thr[k] is the largest float32 x with |x - T[k]| <= |x - T[k+1]|,
// i.e. the exact midpoint (T[k] + T[k+1]) / 2 (exact in double) rounded toward
// minus infinity to float32.  Counting the thresholds that a normalized value
// exceeds gives the nearest level with ties going to the lower index, for every
// float32 input.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "common.hpp"

namespace qlora {
namespace {

double normal_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

double normal_pdf(double x) { return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI); }

// Quantile of N(0,1) for p in (0, 1).
double normal_quantile(double p) {
  double x = 0.0;
  // Newton from 0 converges monotonically for these p (|x| < 2.2); iterate to
  // a fixed point in double precision.
  for (int it = 0; it < 100; ++it) {
    const double f = normal_cdf(x) - p;
    const double step = f / normal_pdf(x);
    x -= step;
    if (std::fabs(step) <= 1e-17 * std::max(1.0, std::fabs(x))) break;
  }
  return x;
}

// thr[k] from the levels: the exact midpoint, rounded toward minus infinity
void set_thresholds(Nf4Table& t) {
  for (int k = 0; k < 15; ++k) {
    const double m = ((double)t.level[k] + (double)t.level[k + 1]) * 0.5;  // exact
    float f = (float)m;
    if ((double)f > m) f = std::nextafter(f, -INFINITY);
    t.thr[k] = f;
  }
}

Nf4Table build_uniform_table() {
  Nf4Table t;
  for (int i = 0; i < 16; ++i) t.level[i] = (float)(-1.0 + 2.0 * i / 15.0);
  set_thresholds(t);
  return t;
}

Nf4Table build_table() {
  std::vector<double> neg, pos;
  for (int j = 0; j < 7; ++j) neg.push_back(normal_quantile((j + 0.5) / 14.0));
  for (int j = 0; j < 8; ++j) pos.push_back(normal_quantile(0.5 + (j + 0.5) / 16.0));
  double neg_scale = 0.0, pos_scale = 0.0;
  for (double v : neg) neg_scale = std::max(neg_scale, std::fabs(v));
  for (double v : pos) pos_scale = std::max(pos_scale, v);
  std::vector<double> lv;
  for (double v : neg) lv.push_back(v / neg_scale);
  lv.push_back(0.0);
  for (double v : pos) lv.push_back(v / pos_scale);
  std::sort(lv.begin(), lv.end());

  Nf4Table t;
  for (int i = 0; i < 16; ++i) t.level[i] = (float)lv[i];
  set_thresholds(t);
  return t;
}

// Bucket tables of the quantization kernel (layout and use: QuantLut).
QuantLut build_lut(const Nf4Table& t, bool* ok) {
  QuantLut L{};
  *ok = true;
  auto bf16_value = [](uint32_t hi16) {
    const uint32_t bits = hi16 << 16;
    float f;
    std::memcpy(&f, &bits, 4);
    return (double)f;
  };
  const double widen = std::ldexp(1.0, -19), floor_abs = std::ldexp(1.0, -140);
  for (int sign = 0; sign < 2; ++sign) {
    for (int idx = 0; idx < kLutSide; ++idx) {
      double mlo, mhi;
      if (idx == 0) {
        mlo = 0.0;
        mhi = std::ldexp(1.0, -6);
      } else {
        mlo = bf16_value(0x3C7Fu + (uint32_t)idx);
        mhi = bf16_value(0x3C7Fu + (uint32_t)idx + 1);
      }
      double lo = sign ? -mhi : mlo, hi = sign ? -mlo : mhi;
      lo -= std::fabs(lo) * widen + floor_abs;
      hi += std::fabs(hi) * widen + floor_abs;
      int below = 0, inside = 0;
      for (int k = 0; k < 15; ++k) {
        if ((double)t.thr[k] < lo) ++below;
        else if ((double)t.thr[k] <= hi) ++inside;
      }
      if (inside > 1) *ok = false;
      L.kidx[sign * kLutSide + idx] = (uint8_t)below;
    }
  }
  for (int k = 0; k < 15; ++k)
    L.mid[k] = ((double)t.thr[k] + (double)std::nextafter(t.thr[k], INFINITY)) * 0.5;  // exact
  L.mid[15] = INFINITY;
  return L;
}

}  // namespace

const Nf4Table& nf4_table() {
  static const Nf4Table table = build_table();
  return table;
}

const Nf4Table& level_table(int table) {
  static const Nf4Table uniform = build_uniform_table();
  return table == kTableUniform ? uniform : nf4_table();
}

const QuantLut& quant_lut(int table, bool* ok) {
  static bool good_nf4 = false, good_uniform = false;
  static const QuantLut lut_nf4 = build_lut(nf4_table(), &good_nf4);
  static const QuantLut lut_uniform = build_lut(level_table(kTableUniform), &good_uniform);
  if (table == kTableUniform) {
    *ok = good_uniform;
    return lut_uniform;
  }
  *ok = good_nf4;
  return lut_nf4;
}

}  // namespace qlora
