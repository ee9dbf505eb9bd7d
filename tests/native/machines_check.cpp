// The split state machines of the HIP path (bit-parallel, bbpe_machines.h)
// against the byte-at-a-time rules they stand for, on random masks with runs.
// Built with the host compiler and run by tests/test_machines.py.
#include <cstdio>
#include <cstdint>
#include <random>
#include <cstdlib>
#include "bbpe_machines.h"
using namespace bbpe;
static uint64_t bit(int i) { return 1ull << i; }
std::mt19937_64 rng(1);
// random mask with runs: density p, mean run length L
uint64_t runs(double p, int L) {
  uint64_t m = 0; int i = 0;
  std::uniform_real_distribution<double> u(0, 1);
  while (i < 64) {
    int len = 1 + int(rng() % (2 * L));
    bool on = u(rng) < p;
    for (int k = 0; k < len && i < 64; ++k, ++i) if (on) m |= bit(i);
  }
  return m;
}
uint64_t sparse(double p) { uint64_t m = 0; std::uniform_real_distribution<double> u(0,1); for (int i = 0; i < 64; ++i) if (u(rng) < p) m |= bit(i); return m; }

int main(int argc, char **argv) {
  const long iters = argc > 1 ? atol(argv[1]) : 200000;
  long bad = 0, n = 0;
  for (long it = 0; it < iters; ++it) {
    // ---- digits (single-byte digits: N_ == DL)
    uint64_t N_ = runs(0.4, 1 + it % 7), SS = sparse(it % 3 ? 0.02 : 0.2);
    uint64_t pNin = rng() & 1;  // previous byte digit?
    uint64_t pN = (N_ << 1) | pNin;
    uint64_t DL = N_;
    uint64_t RS = DL & (SS | ~pN);
    uint32_t ph_in = pNin ? uint32_t(rng() % 3) : 3u;
    if (it % 11 == 0) ph_in = uint32_t(rng() % 4);
    // reference
    uint64_t PH0 = 0; uint32_t ph = ph_in;
    for (int i = 0; i < 64; ++i) { uint64_t b = bit(i);
      if (DL & b) { ph = (RS & b) ? 0u : (ph == 3u ? 0u : (ph + 1u) % 3u); if (ph == 0) PH0 |= b; }
      else if (!(N_ & b)) ph = 3; }
    uint64_t got = digit_phase0_ascii(DL, RS, ph_in);
    ++n; if (got != PH0) { if (bad++ < 5) printf("digit PH0 N=%016lx RS=%016lx ph_in=%u ref=%016lx got=%016lx\n", N_, RS, ph_in, PH0, got); }
    // phase out, general (multi-byte digits too): LD sparse within N_
    uint64_t N2 = runs(0.5, 1 + it % 9), LD2 = N2 & (it % 2 ? ~0ull : sparse(0.5)) ;
    uint64_t DL2 = N2 & LD2; uint64_t SS2 = sparse(0.05); uint64_t pN2 = (N2 << 1) | (rng() & 1);
    uint64_t RS2 = DL2 & (SS2 | ~pN2);
    if (!(N2 == ~0ull && RS2 == 0)) {
      uint32_t p2 = 3;
      for (int i = 0; i < 64; ++i) { uint64_t b = bit(i);
        if (N2 & LD2 & b) p2 = (RS2 & b) ? 0u : (p2 == 3u ? 0u : (p2 + 1u) % 3u);
        else if (!(N2 & b)) p2 = 3; }
      uint32_t g2 = digit_phase_out(N2, DL2, RS2);
      ++n; if (g2 != p2) { if (bad++ < 5) printf("digit out N=%016lx LD=%016lx RS=%016lx ref=%u got=%u\n", N2, LD2, RS2, p2, g2); }
    }
    // ---- CR runs
    uint64_t IN = ~sparse(it % 5 ? 0.0 : 0.1);
    uint64_t CR_ = runs(0.3, 1 + it % 4) & IN;
    uint64_t SS3 = sparse(it % 4 ? 0.03 : 0.3);
    uint64_t pO = sparse(0.3), NC = runs(0.4, 2) & ~CR_, LD = ~sparse(0.2);
    uint32_t st_in = uint32_t(rng() % 3);
    uint64_t E2ref = 0; uint32_t st = st_in;
    for (int i = 0; i < 64; ++i) { uint64_t b = bit(i);
      if (!(IN & b)) st = 0;
      else if (CR_ & b) st = (SS3 & b) ? 2u : (st == 0 ? ((pO & b) ? 1u : 2u) : st);
      else { if (st == 1 && (NC & LD & b) && !(SS3 & b)) E2ref |= b; st = 0; } }
    uint64_t E2; uint32_t so = cr_runs(CR_, IN, SS3, pO, NC & LD, st_in, E2);
    ++n; if (E2 != E2ref || so != st) { if (bad++ < 5) printf("cr CR=%016lx IN=%016lx SS=%016lx pO=%016lx st_in=%u ref E2=%016lx st=%u got %016lx %u\n", CR_, IN, SS3, pO, st_in, E2ref, st, E2, so); }
    // ---- v machine
    uint64_t BRK = sparse(it % 3 ? 0.02 : 0.2), NCv = runs(0.5, 1 + it % 6), WS = NCv | sparse(0.2);
    uint32_t v = uint32_t(rng() & 1), vin = v;
    uint64_t VNref = 0;
    for (int i = 63; i >= 0; --i) { uint64_t b = bit(i);
      if (v) VNref |= b;
      if (BRK & b) v = 0; else if (NCv & b) {} else v = (WS & b) ? 0u : 1u; }
    uint64_t VN = v_next(BRK, NCv, WS, vin);
    ++n; if (VN != VNref) { if (bad++ < 5) printf("v BRK=%016lx NC=%016lx WS=%016lx vin=%u ref=%016lx got=%016lx\n", BRK, NCv, WS, vin, VNref, VN); }
  }
  printf("checked %ld, mismatches %ld\n", n, bad);
  return bad != 0;
}
