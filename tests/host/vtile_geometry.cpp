// Host check of the attention forward's transposing value-tile reads, for
// every head dim and 16-bit type the forward takes: simulates
// ds_read_b64_tr_b16 on the addresses vt_read_offset gives each lane and
// checks that (1) every lane receives, in its four values, the keys its
// MFMA k slots stand for (keys 16c + 8*half + 4*(lane/32) + m) of its own
// output column (dg*32 + lane%32), a column past the head dim landing in the
// row's zero padding; (2) every read is 8-byte aligned and inside the tile;
// (3) within each half wave no two different dwords share one of the 64
// four-byte LDS banks.
//
// The lane rule of the instruction, measured on the GPU with index-coded LDS
// contents: within each group of 16 lanes, lane i receives as its value m
// (m = 0..3) value i % 4 of the 8-byte unit that lane i/4 + 4m of its group
// addresses.
#include <cstdio>
#include <map>

#include "vtile.h"

using namespace tsel;

template <int DT, int D>
static int check() {
  using VG = VGeom<DT, D>;
  constexpr int DG = OGroups<D>::DG, ES = VG::ES, RS = VG::RS;
  if (DG * 32 * ES > RS) {
    std::printf("FAIL D=%d: padded columns leave the row\n", D);
    return 1;
  }
  for (int dg = 0; dg < DG; ++dg)
    for (int c = 0; c < 2; ++c)
      for (int half = 0; half < 2; ++half) {
        int addr[64];
        for (int lane = 0; lane < 64; ++lane) {
          addr[lane] = vt_read_offset<DT, D>(lane, dg, c, half);
          if (addr[lane] < 0 || addr[lane] % 8 != 0 || addr[lane] + 8 > VG::TILE) {
            std::printf("FAIL D=%d dg=%d c=%d half=%d lane %d: address %d (tile %d bytes)\n", D, dg, c, half,
                        lane, addr[lane], VG::TILE);
            return 1;
          }
        }
        for (int h = 0; h < 2; ++h) {
          std::map<int, int> bank_dword;
          for (int lane = 32 * h; lane < 32 * h + 32; ++lane)
            for (int w = 0; w < 2; ++w) {
              const int dw = addr[lane] / 4 + w, bank = dw % 64;
              auto it = bank_dword.find(bank);
              if (it != bank_dword.end() && it->second != dw) {
                std::printf("FAIL D=%d dg=%d c=%d half=%d: bank %d holds dwords %d and %d\n", D, dg, c, half,
                            bank, it->second, dw);
                return 1;
              }
              bank_dword[bank] = dw;
            }
        }
        for (int lane = 0; lane < 64; ++lane) {
          const int g = lane / 16, i = lane % 16;
          for (int m = 0; m < 4; ++m) {
            const int src = 16 * g + i / 4 + 4 * m;
            const int byte = addr[src] + (i % 4) * ES;
            const int row = byte / RS, col = (byte % RS) / ES;
            const int want_row = 16 * c + 8 * half + 4 * (lane / 32) + m, want_col = dg * 32 + lane % 32;
            const bool pad_ok = want_col >= D && col * ES >= VG::UNITS_D * 16;
            if (row != want_row || col != want_col || (want_col >= D && !pad_ok)) {
              std::printf("FAIL D=%d dg=%d c=%d half=%d lane %d value %d: row %d col %d, want row %d col %d\n",
                          D, dg, c, half, lane, m, row, col, want_row, want_col);
              return 1;
            }
          }
        }
      }
  return 0;
}

int main() {
  int bad = 0;
  bad |= check<TSEL_BF16, 64>() | check<TSEL_BF16, 72>() | check<TSEL_BF16, 80>() | check<TSEL_BF16, 96>() |
         check<TSEL_BF16, 128>();
  bad |= check<TSEL_F16, 64>() | check<TSEL_F16, 72>() | check<TSEL_F16, 80>() | check<TSEL_F16, 96>() |
         check<TSEL_F16, 128>();
  if (bad) return 1;
  std::printf("ok\n");
  return 0;
}
