// Decode step: launch of the 8-bit-state kernels (the kernels themselves
// are templates in decode_impl.h).
#include <atomic>
#include <cstdlib>

#include "decode_impl.h"

namespace gdnq {

namespace {
int env_int(const char* name) {
  const char* e = std::getenv(name);
  const long v = e ? std::atol(e) : 0;
  return v > 0 && v < (1L << 30) ? int(v) : 0;
}
std::atomic<int> g_grid{env_int("GDNQ_DECODE_GRID")};
std::atomic<int> g_open_waves{env_int("GDNQ_DECODE_OPEN_WAVES")};
}  // namespace

DecodeSchedule decode_schedule() {
  return {g_grid.load(std::memory_order_relaxed), g_open_waves.load(std::memory_order_relaxed)};
}

void set_decode_schedule(int grid, int open_waves) {
  g_grid.store(grid > 0 && grid < (1 << 30) ? grid : 0, std::memory_order_relaxed);
  g_open_waves.store(open_waves > 0 && open_waves < (1 << 30) ? open_waves : 0, std::memory_order_relaxed);
}

int decode_row_split() { return 8; }  // close jobs per head at most (grid validation)
int decode_max_batch() { return DEC_MAXB; }
hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream) {
  if (L.sliding) return launch_decode_sliding(L, stream);
  DecodeArgs a{L.q,        L.k,        L.v,       L.alpha,   L.beta,   L.codes, L.scales, L.buf_k,
               L.buf_v,    L.buf_alpha, L.buf_beta, L.fill_in, L.fill_out, L.o,   L.B,      L.H,
               L.W,        decode_open_waves(), nullptr,   nullptr};
  if (L.buf_fp8) {  // the per-vector scales follow the codes in each buffer
    const size_t nv = size_t(L.B) * L.H * L.W;
    a.ks = reinterpret_cast<float*>(static_cast<char*>(L.buf_k) + nv * L.d_k);
    a.vs = reinterpret_cast<float*>(static_cast<char*>(L.buf_v) + nv * L.d_v);
  }
  return L.q4 ? launch_decode_q4(L, a, stream) : launch_qb<8>(L, a, stream);
}

}  // namespace gdnq
