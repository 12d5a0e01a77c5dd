// Offline encoder of the trellis-coded middle tier (host code).
//
// SpAx page, section 5.1 (trellis coding): every column becomes a sequence of
// 2-bit codes and one scale, its root-mean-square; weight i is read through
// the window of the codes of rows i-7..i, a 16-bit index into a shared
// codebook of 2^16 values, times the scale; codes before the column start
// are zero; the codes minimise the total squared error between the
// normalised weights and their reconstructions, chosen jointly with the
// Viterbi algorithm. The encoder runs once, offline, on the host.
//
// Fixed here so that every encoder gives the same codes:
//   * window: index_i = (index_{i-1} >> 2) | (c_i << 14) (oldest code in the
//     low bits); the trellis state after row i is index_i >> 2, so state t
//     at row i comes from state ((t & 0xFFF) << 2) | o through index 4t + o;
//   * scale: S = sum of w_i^2 as an exact integer in units of 2^-48, then
//     fp16(sqrt(fp64(fp64(S) / R)) 2^-24), each step rounded once;
//   * errors in fp32, each operation rounded (this file is compiled without
//     floating-point contraction): v_i = fp32(w_i / s), d = v_i - cb,
//     e = d * d, cost' = cost + e; the smallest o wins ties, the smallest
//     final state wins ties; a zero column gets scale 0 and zero codes.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <limits>
#include <new>
#include <thread>
#include <utility>
#include <vector>

#include "spax.h"

namespace {

double h2d(uint16_t b) {
  const int e = (b >> 10) & 31, m = b & 1023;
  const double mag = e == 0 ? std::ldexp((double)m, -24) : std::ldexp((double)(m | 1024), e - 25);
  return (b & 0x8000u) ? -mag : mag;
}

// fp16 value as an integer in units of 2^-24 (finite values)
int64_t h_units(uint16_t b) {
  const uint32_t e = (b >> 10) & 31u, m = b & 1023u;
  const int64_t mag = e == 0u ? (int64_t)m : (int64_t)(m | 1024u) << (e - 1u);
  return (b & 0x8000u) ? -mag : mag;
}

// round a finite v >= 0 to fp16, ties to even, in one step
uint16_t d2h_rne(double v) {
  if (v == 0.0) return 0;
  int e;
  (void)std::frexp(v, &e);  // v in [2^(e-1), 2^e)
  int E = e - 1;
  if (E < -14) return (uint16_t)std::nearbyint(std::ldexp(v, 24));
  uint32_t q = (uint32_t)std::nearbyint(std::ldexp(v, 10 - E));
  if (q == 2048u) {
    q = 1024u;
    ++E;
  }
  if (E > 15) return 0x7C00;
  return (uint16_t)(((uint32_t)(E + 15) << 10) | (q - 1024u));
}

constexpr int kStates = 1 << 14;

void encode_column(const uint16_t* w, int R, const float* cb, uint8_t* codes, uint16_t* scale,
                   std::vector<float>& cost, std::vector<float>& next,
                   std::vector<uint8_t>& back) {
  unsigned __int128 S = 0;
  for (int i = 0; i < R; ++i) {
    const int64_t u = h_units(w[i]);
    S += (unsigned __int128)((__int128)u * u);
  }
  const double q = (double)S / (double)R;
  const uint16_t sh = d2h_rne(std::ldexp(std::sqrt(q), -24));
  *scale = sh;
  for (int b = 0; b < R / 4; ++b) codes[b] = 0;
  if (sh == 0) return;
  const double s = h2d(sh);
  const float inf = std::numeric_limits<float>::infinity();
  for (int t = 0; t < kStates; ++t) cost[t] = inf;
  cost[0] = 0.0f;
  for (int i = 0; i < R; ++i) {
    const float v = (float)(h2d(w[i]) / s);
    uint8_t* bk = back.data() + (size_t)i * kStates;
    for (int t = 0; t < kStates; ++t) {
      const int p0 = (t & 0xFFF) << 2;
      float best = 0.0f;
      int bo = 0;
      for (int o = 0; o < 4; ++o) {
        const float d = v - cb[4 * t + o];
        const float e = d * d;
        const float c = cost[p0 | o] + e;
        if (o == 0 || c < best) {
          best = c;
          bo = o;
        }
      }
      next[t] = best;
      bk[t] = (uint8_t)bo;
    }
    cost.swap(next);
  }
  int state = 0;
  for (int t = 1; t < kStates; ++t)
    if (cost[t] < cost[state]) state = t;
  for (int i = R - 1; i >= 0; --i) {
    const uint32_t c = (uint32_t)state >> 12;
    codes[i >> 2] |= (uint8_t)(c << (2 * (i & 3)));
    state = ((state & 0xFFF) << 2) | back[(size_t)i * kStates + state];
  }
}

}  // namespace

extern "C" int spax_pack_trellis_host(const uint16_t* w, int32_t rows, int32_t cols,
                                      const uint16_t* codebook, uint8_t* codes,
                                      uint16_t* scales, int32_t threads) {
  if (!w || !codebook || !codes || !scales) return SPAX_ENULL;
  if (rows <= 0 || cols <= 0 || rows % 128 || rows > (1 << 20)) return SPAX_EINVAL;
  if (threads < 1) threads = 1;
  if (threads > cols) threads = cols;
  // Every allocation happens here, before any thread starts, so that a
  // shortage becomes fewer threads or an error code, never an exception
  // escaping a worker (which would end the process).
  struct Scratch {
    std::vector<float> cost, next;
    std::vector<uint8_t> back;
  };
  std::vector<float> cb;
  std::vector<Scratch> scratch;
  try {
    cb.resize(65536);
    scratch.reserve((size_t)threads);
    for (int k = 0; k < threads; ++k) {
      Scratch sc;
      sc.cost.resize(kStates);
      sc.next.resize(kStates);
      sc.back.resize((size_t)rows * kStates);
      scratch.push_back(std::move(sc));
    }
  } catch (const std::bad_alloc&) {
    if (cb.size() != 65536 || scratch.empty()) return SPAX_ENOMEM;
  }
  for (int k = 0; k < 65536; ++k) cb[k] = (float)h2d(codebook[k]);
  // columns are handed out one at a time, so any number of workers covers
  // all of them
  std::atomic<int> next_col{0};
  auto work = [&](Scratch* sc) {
    for (int j = next_col.fetch_add(1); j < cols; j = next_col.fetch_add(1))
      encode_column(w + (size_t)j * rows, rows, cb.data(), codes + (size_t)j * (rows / 4),
                    scales + j, sc->cost, sc->next, sc->back);
  };
  std::vector<std::thread> pool;
  for (size_t k = 1; k < scratch.size(); ++k) {
    try {
      pool.emplace_back(work, &scratch[k]);
    } catch (const std::exception&) {
      break;  // the threads already started and this one share the columns
    }
  }
  work(&scratch[0]);
  for (auto& th : pool) th.join();
  return SPAX_OK;
}
