// LDS bank model of the exchange layouts (test infrastructure, host only).
//
// For every row length the kernels instantiate, this program lists the LDS
// addresses that each exchange access of the pass schedule touches, thread by
// thread, using the layout functions of rdfft_device.hpp itself (Row<P, E>:
// stride, addr, the item order of each pass).  The accesses are those of the
// forward (pass-0 scatter; each later pass's gather and scatter, the last one
// into the natural order; the staged store's reads) and of the inverse (each
// pass's scatter and gather down to the final read of layout E).  It also
// lists the load loop of the 2D column tiles (ColShape<H>).
//
// Cost of one access, per wavefront: each 32-lane half takes as many cycles as
// the largest number of distinct addresses that fall in one of the 32 banks
// (a bank holds address mod 32); extra cycles = that sum minus 2.  Rows
// shorter than a wavefront sit Row::LDS floats apart, as in the kernels.
// Against rocprofv3's SQ_LDS_BANK_CONFLICT this count is exact: 1024 and 37888
// extra cycles per row at p = 16384 and 32768 (1.05M and 19.4M per launch of
// 1024 and 512 rows) before the layout at 32768 was changed, and 3072 per load
// loop of a 4096-row column tile before its stride was changed.
//
// Output, one line each:
//   row <P> <E> <fwd extra cycles per row> <inv extra cycles per row>
//   col <H> <CL> <CS> <extra cycles per tile load loop>
#include <cstdio>
#include <set>
#include <vector>

#include "rdfft2d_kernels.hpp"

using namespace rdfft;

namespace {

// extra cycles of one access; addr[l] for the 64 lanes
long wave_extra(const std::vector<long>& a) {
  long extra = 0;
  for (int h = 0; h < 2; ++h) {
    std::set<long> per[32];
    for (int l = 32 * h; l < 32 * h + 32; ++l) per[((a[l] % 32) + 32) % 32].insert(a[l]);
    size_t worst = 0;
    for (auto& s : per) worst = s.size() > worst ? s.size() : worst;
    extra += static_cast<long>(worst) - 1;
  }
  return extra;
}

template <int P, int E>
struct Model {
  using Rw = Row<P, E>;
  static constexpr int T = Rw::T;
  std::vector<std::vector<long>> acc;  // per access: address of each thread t of a row

  template <class F>
  void add(F f) {
    std::vector<long> a(T);
    for (int t = 0; t < T; ++t) a[t] = f(t);
    acc.push_back(a);
  }

  // forward pass with input size B: gathers from layout B, scatter to layout B*R
  template <int B>
  void fwd_from() {
    using PS = typename Rw::template Pass<B>;
    constexpr int R = PS::R, LR = ilog2(R);
    for (int n = 0; n < PS::IPT; ++n)
      for (int q = 0; q < R; ++q)
        for (int half = 0; half < 2; ++half)
          add([&](int t) {
            int rp, k;
            PS::item(t + T * n, rp, k);
            const int k2 = (k == 0) ? (B / 2) : (B - k);
            return Rw::template addr<B>(rp + PS::NRES * bitrev(q, LR), half ? k2 : k);
          });
    for (int n = 0; n < PS::IPT; ++n)
      for (int q = 0; q < R; ++q)
        for (int half = 0; half < 2; ++half)
          add([&](int t) {
            int rp, k;
            PS::item(t + T * n, rp, k);
            const int k2 = (k == 0) ? (B / 2) : (B - k);
            return Rw::template addr<PS::BP>(rp, q * B + (half ? k2 : k));
          });
    if constexpr (PS::BP != P) fwd_from<PS::BP>();
  }

  void forward() {
    for (int s = 0; s < E; ++s) add([&](int t) { return Rw::template addr<E>(t, s); });
    fwd_from<E>();
    for (int s = 0; s < E; ++s) add([&](int t) { return t + T * s; });  // staged store
  }

  // inverse pass with input size B: scatter to layout B (after its gather
  // from layout B*R, which the first pass takes from HBM instead)
  template <int B>
  void inv_scatter() {
    using PS = typename Rw::template Pass<B>;
    constexpr int R = PS::R, LR = ilog2(R);
    for (int n = 0; n < PS::IPT; ++n)
      for (int q = 0; q < R; ++q)
        for (int half = 0; half < 2; ++half)
          add([&](int t) {
            int rp, k;
            PS::item(t + T * n, rp, k);
            const int k2 = (k == 0) ? (B / 2) : (B - k);
            return Rw::template addr<B>(rp + PS::NRES * bitrev(q, LR), half ? k2 : k);
          });
  }
  template <int B>
  void inv_gather() {
    using PS = typename Rw::template Pass<B>;
    for (int n = 0; n < PS::IPT; ++n)
      for (int q = 0; q < PS::R; ++q)
        for (int half = 0; half < 2; ++half)
          add([&](int t) {
            int rp, k;
            PS::item(t + T * n, rp, k);
            const int k2 = (k == 0) ? (B / 2) : (B - k);
            return Rw::template addr<PS::BP>(rp, half ? k2 : k) + q * B;
          });
  }
  template <int Bout>
  void inv_down() {
    if constexpr (Bout > E) {
      constexpr int B = Rw::pass_in_for(Bout);
      inv_gather<B>();
      inv_scatter<B>();
      inv_down<B>();
    }
  }

  void inverse() {
    constexpr int BL = Rw::pass_in_for(P);
    inv_scatter<BL>();
    inv_down<BL>();
    for (int s = 0; s < E; ++s) add([&](int t) { return Rw::template addr<E>(t, s); });
  }

  // extra cycles per row over all accesses
  double cost() const {
    const int rows_per_wave = T >= 64 ? 1 : 64 / T;
    const int waves = T >= 64 ? T / 64 : 1;
    long total = 0;
    for (const auto& a : acc)
      for (int w = 0; w < waves; ++w) {
        std::vector<long> lanes(64);
        for (int l = 0; l < 64; ++l)
          lanes[l] = T >= 64 ? a[64 * w + l] : (l / T) * static_cast<long>(Rw::LDS) + a[l % T];
        total += wave_extra(lanes);
      }
    return static_cast<double>(total) / rows_per_wave;
  }
};

template <int P, int E>
void row_line() {
  Model<P, E> f, i;
  f.forward();
  i.inverse();
  std::printf("row %d %d %g %g\n", P, E, f.cost(), i.cost());
}

template <int H>
void col_line() {
  using S = ColShape<H>;
  long total = 0;
  for (int w = 0; w < S::NT / 64; ++w)
    for (int i = 0; i < H * S::CL; i += S::NT) {
      std::vector<long> lanes(64);
      for (int l = 0; l < 64; ++l) {
        const int e = 64 * w + l + i;
        lanes[l] = static_cast<long>(e % S::CL) * S::CS + e / S::CL;
      }
      total += wave_extra(lanes);
    }
  std::printf("col %d %d %d %ld\n", H, S::CL, S::CS, total);
}

}  // namespace

int main() {
  row_line<32, 16>();
  row_line<64, 16>();
  row_line<128, 16>();
  row_line<256, 16>();
  row_line<512, 16>();
  row_line<1024, 16>();
  row_line<2048, 16>();
  row_line<4096, 16>();
  row_line<8192, 16>();
  row_line<16384, long_elems(16384)>();
  row_line<32768, long_elems(32768)>();
  col_line<32>();
  col_line<64>();
  col_line<128>();
  col_line<256>();
  col_line<512>();
  col_line<1024>();
  col_line<2048>();
  col_line<4096>();
  return 0;
}
