// Host driver of the LDS schedule checker: the library's C ABI (rdfft_lib.hip,
// built for the host against the CPU stand-in of hip/hip_runtime.h) called on
// host buffers read from and written to raw little-endian files.
//
//   run_abi fwd|inv    <rows> <p> <dtype> <data>
//   run_abi fwd2d|inv2d <n> <h> <w> <dtype> <data>
//   run_abi unpack     <rows> <p> <dtype> <packed> <spec>
//   run_abi pack       <rows> <p> <dtype> <spec> <packed>
//   run_abi circ_fwd   <batch> <d_in> <d_out> <p> <dtype> <x> <c> <y>
//   run_abi circ_bwd   <batch> <d_in> <d_out> <p> <dtype> <x> <c> <dy> <dx|-> <dc|->
//   run_abi circ_det   <batch> <d_in> <d_out> <p> <dtype> <x> <c> <dy> <dx|-> <dc>
//                      (circulant_bwd_det with a workspace of the size its query
//                      gives, filled with garbage; dc filled with garbage too)
//   run_abi circ_step  <batch> <d_in> <d_out> <p> <dtype> <x> <c> <dy> <y> <dx|-> <dc>
//                      (circulant_fwd_zero into a dc that holds garbage, then
//                      circulant_bwd_acc twice: dc = 2 x the gradient)
//   run_abi circ_spec  <batch> <d_in> <d_out> <p> <dtype> <x> <c> <dy> <y> <y2> <dx|-> <dc> <cs>
//                      (the weights given as spectra: circulant_fwd_step
//                      writing y and cs and clearing a dc that holds garbage;
//                      circulant_weight_spectra into a second buffer, which
//                      must equal cs bitwise; circulant_fwd_spec from it into
//                      y2; then circulant_bwd_spec overwriting dc and once
//                      more adding into it: dc = 2 x the gradient)
//   run_abi cases      (stdin: one call per line, "<entry point> <arg> ...", a
//                      pointer argument as an integer address or "null"; prints
//                      each call's status, one per line)
//   run_abi selftest race|ok   (a 64-thread kernel whose threads exchange LDS
//                      values without / with a barrier in between: the
//                      sanitizer must report the first and not the second)
//
// dtype is 0 (fp32), 1 (bf16) or 2 (fp16), as in rdfft.h; c, dc and spectra
// are fp32.  In-place data is read and written back to the same file; an
// output that is also listed as input ("-" skips it) is created.  Exit status
// 0 with "status <s> launches <l> workgroups <w>" on stdout.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "rdfft_lib.hip"

namespace {

struct Buf {
  void* p = nullptr;
  size_t n = 0;
};

Buf alloc(size_t n) {
  Buf b;
  b.n = n;
  b.p = std::aligned_alloc(64, (n + 63) / 64 * 64 + 64);
  std::memset(b.p, 0, (n + 63) / 64 * 64 + 64);
  return b;
}

Buf read_file(const char* path, size_t n) {
  Buf b = alloc(n);
  FILE* f = std::fopen(path, "rb");
  if (!f || std::fread(b.p, 1, n, f) != n) {
    std::fprintf(stderr, "cannot read %zu bytes from %s\n", n, path);
    std::exit(2);
  }
  std::fclose(f);
  return b;
}

void write_file(const char* path, const Buf& b) {
  FILE* f = std::fopen(path, "wb");
  if (!f || std::fwrite(b.p, 1, b.n, f) != b.n) {
    std::fprintf(stderr, "cannot write %s\n", path);
    std::exit(2);
  }
  std::fclose(f);
}

int64_t arg(char** argv, int i) { return std::strtoll(argv[i], nullptr, 10); }

__global__ void selftest_kernel(float* out, int barrier) {
  __shared__ float s[64];
  s[threadIdx.x] = static_cast<float>(threadIdx.x);
  if (barrier) __syncthreads();
  out[threadIdx.x] = s[(threadIdx.x + 1) % 64];
}

// one line of the "cases" op: the entry point and its arguments (no stream)
int call_case(const std::string& line) {
  std::vector<std::string> tok;
  size_t i = 0;
  while (i < line.size()) {
    while (i < line.size() && line[i] == ' ') ++i;
    size_t j = i;
    while (j < line.size() && line[j] != ' ') ++j;
    if (j > i) tok.push_back(line.substr(i, j - i));
    i = j;
  }
  if (tok.empty()) return -100;
  auto ptr = [&](size_t k) -> void* {
    return tok[k] == "null" ? nullptr : reinterpret_cast<void*>(static_cast<uintptr_t>(std::stoull(tok[k])));
  };
  auto num = [&](size_t k) -> int64_t { return std::stoll(tok[k]); };
  const std::string& f = tok[0];
  const size_t n = tok.size() - 1;
  if ((f == "rdfft_forward" || f == "rdfft_inverse") && n == 4)
    return (f == "rdfft_forward" ? rdfft_forward : rdfft_inverse)(ptr(1), num(2), num(3), int(num(4)), nullptr);
  if ((f == "rdfft2d_forward" || f == "rdfft2d_inverse") && n == 5)
    return (f == "rdfft2d_forward" ? rdfft2d_forward : rdfft2d_inverse)(ptr(1), num(2), num(3), num(4),
                                                                        int(num(5)), nullptr);
  if (f == "rdfft_unpack" && n == 5)
    return rdfft_unpack(ptr(1), static_cast<float*>(ptr(2)), num(3), num(4), int(num(5)), nullptr);
  if (f == "rdfft_pack" && n == 5)
    return rdfft_pack(static_cast<const float*>(ptr(1)), ptr(2), num(3), num(4), int(num(5)), nullptr);
  if (f == "circulant_fwd" && n == 8)
    return circulant_fwd(ptr(1), static_cast<const float*>(ptr(2)), ptr(3), num(4), num(5), num(6), num(7),
                         int(num(8)), nullptr);
  if (f == "circulant_fwd_zero" && n == 9)
    return circulant_fwd_zero(ptr(1), static_cast<const float*>(ptr(2)), ptr(3), static_cast<float*>(ptr(4)), num(5),
                              num(6), num(7), num(8), int(num(9)), nullptr);
  if (f == "circulant_bwd_acc" && n == 10)
    return circulant_bwd_acc(ptr(1), static_cast<const float*>(ptr(2)), ptr(3), ptr(4), static_cast<float*>(ptr(5)),
                             num(6), num(7), num(8), num(9), int(num(10)), nullptr);
  if (f == "circulant_bwd_det" && n == 12)
    return circulant_bwd_det(ptr(1), static_cast<const float*>(ptr(2)), ptr(3), ptr(4), static_cast<float*>(ptr(5)),
                             static_cast<float*>(ptr(6)), num(7), num(8), num(9), num(10), num(11), int(num(12)),
                             nullptr);
  if (f == "circulant_bwd_det_noalloc" && n == 10)
    return circulant_bwd_det_noalloc(ptr(1), static_cast<const float*>(ptr(2)), ptr(3), ptr(4),
                                     static_cast<float*>(ptr(5)), num(6), num(7), num(8), num(9), int(num(10)),
                                     nullptr);
  if (f == "circulant_bwd_det_workspace" && n == 6)
    return circulant_bwd_det_workspace(num(1), num(2), num(3), num(4), int(num(5)),
                                       static_cast<int64_t*>(ptr(6)));
  if (f == "circulant_weight_spectra" && n == 5)
    return circulant_weight_spectra(static_cast<const float*>(ptr(1)), static_cast<float*>(ptr(2)), num(3), num(4),
                                    num(5), nullptr);
  if (f == "circulant_fwd_step" && n == 10)
    return circulant_fwd_step(ptr(1), static_cast<const float*>(ptr(2)), ptr(3), static_cast<float*>(ptr(4)),
                              static_cast<float*>(ptr(5)), num(6), num(7), num(8), num(9), int(num(10)), nullptr);
  if (f == "circulant_fwd_spec" && n == 9)
    return circulant_fwd_spec(ptr(1), static_cast<const float*>(ptr(2)), ptr(3), static_cast<float*>(ptr(4)), num(5),
                              num(6), num(7), num(8), int(num(9)), nullptr);
  if (f == "circulant_bwd_spec" && n == 11)
    return circulant_bwd_spec(ptr(1), static_cast<const float*>(ptr(2)), ptr(3), ptr(4), static_cast<float*>(ptr(5)),
                              int(num(6)), num(7), num(8), num(9), num(10), int(num(11)), nullptr);
  if (f == "circulant_bwd" && n == 10)
    return circulant_bwd(ptr(1), static_cast<const float*>(ptr(2)), ptr(3), ptr(4), static_cast<float*>(ptr(5)),
                         num(6), num(7), num(8), num(9), int(num(10)), nullptr);
  return -100;
}
size_t esize(int dtype) { return dtype == RDFFT_F32 ? 4 : 2; }

}  // namespace

int main(int argc, char** argv) {
  if (argc < 2) return 2;
  const std::string op = argv[1];
  int st = -1;
  if ((op == "fwd" || op == "inv") && argc == 6) {
    const int64_t rows = arg(argv, 2), p = arg(argv, 3);
    const int dt = static_cast<int>(arg(argv, 4));
    Buf d = read_file(argv[5], rows * p * esize(dt));
    st = op == "fwd" ? rdfft_forward(d.p, rows, p, dt, nullptr) : rdfft_inverse(d.p, rows, p, dt, nullptr);
    write_file(argv[5], d);
  } else if ((op == "fwd2d" || op == "inv2d") && argc == 7) {
    const int64_t n = arg(argv, 2), h = arg(argv, 3), w = arg(argv, 4);
    const int dt = static_cast<int>(arg(argv, 5));
    Buf d = read_file(argv[6], n * h * w * esize(dt));
    st = op == "fwd2d" ? rdfft2d_forward(d.p, n, h, w, dt, nullptr) : rdfft2d_inverse(d.p, n, h, w, dt, nullptr);
    write_file(argv[6], d);
  } else if (op == "unpack" && argc == 7) {
    const int64_t rows = arg(argv, 2), p = arg(argv, 3);
    const int dt = static_cast<int>(arg(argv, 4));
    Buf z = read_file(argv[5], rows * p * esize(dt));
    Buf s = alloc(rows * (p / 2 + 1) * 2 * 4);
    st = rdfft_unpack(z.p, static_cast<float*>(s.p), rows, p, dt, nullptr);
    write_file(argv[6], s);
  } else if (op == "pack" && argc == 7) {
    const int64_t rows = arg(argv, 2), p = arg(argv, 3);
    const int dt = static_cast<int>(arg(argv, 4));
    Buf s = read_file(argv[5], rows * (p / 2 + 1) * 2 * 4);
    Buf z = alloc(rows * p * esize(dt));
    st = rdfft_pack(static_cast<const float*>(s.p), z.p, rows, p, dt, nullptr);
    write_file(argv[6], z);
  } else if (op == "circ_fwd" && argc == 10) {
    const int64_t b = arg(argv, 2), di = arg(argv, 3), dout = arg(argv, 4), p = arg(argv, 5);
    const int dt = static_cast<int>(arg(argv, 6));
    Buf x = read_file(argv[7], b * di * esize(dt));
    Buf c = read_file(argv[8], (dout / p) * di * 4);
    Buf y = alloc(b * dout * esize(dt));
    st = circulant_fwd(x.p, static_cast<const float*>(c.p), y.p, b, di, dout, p, dt, nullptr);
    write_file(argv[9], y);
  } else if (op == "circ_bwd" && argc == 12) {
    const int64_t b = arg(argv, 2), di = arg(argv, 3), dout = arg(argv, 4), p = arg(argv, 5);
    const int dt = static_cast<int>(arg(argv, 6));
    Buf x = read_file(argv[7], b * di * esize(dt));
    Buf c = read_file(argv[8], (dout / p) * di * 4);
    Buf dy = read_file(argv[9], b * dout * esize(dt));
    const bool want_dx = std::strcmp(argv[10], "-") != 0, want_dc = std::strcmp(argv[11], "-") != 0;
    Buf dx = alloc(b * di * esize(dt));
    Buf dc = alloc((dout / p) * di * 4);
    // dc is overwritten, whatever it held before
    for (size_t i = 0; i < dc.n / 4; ++i) static_cast<float*>(dc.p)[i] = 12345.0f;
    st = circulant_bwd(x.p, static_cast<const float*>(c.p), dy.p, want_dx ? dx.p : nullptr,
                       want_dc ? static_cast<float*>(dc.p) : nullptr, b, di, dout, p, dt, nullptr);
    if (want_dx) write_file(argv[10], dx);
    if (want_dc) write_file(argv[11], dc);
  } else if (op == "circ_det" && argc == 12) {
    const int64_t b = arg(argv, 2), di = arg(argv, 3), dout = arg(argv, 4), p = arg(argv, 5);
    const int dt = static_cast<int>(arg(argv, 6));
    Buf x = read_file(argv[7], b * di * esize(dt));
    Buf c = read_file(argv[8], (dout / p) * di * 4);
    Buf dy = read_file(argv[9], b * dout * esize(dt));
    const bool want_dx = std::strcmp(argv[10], "-") != 0;
    int64_t need = 0;
    st = circulant_bwd_det_workspace(b, di, dout, p, want_dx ? 1 : 0, &need);
    if (st == RDFFT_OK) {
      Buf ws = alloc(static_cast<size_t>(need));
      for (size_t i = 0; i < ws.n / 4; ++i) static_cast<float*>(ws.p)[i] = -777.0f;
      Buf dx = alloc(b * di * esize(dt));
      Buf dc = alloc((dout / p) * di * 4);
      for (size_t i = 0; i < dc.n / 4; ++i) static_cast<float*>(dc.p)[i] = 12345.0f;
      st = circulant_bwd_det(x.p, static_cast<const float*>(c.p), dy.p, want_dx ? dx.p : nullptr,
                             static_cast<float*>(dc.p), static_cast<float*>(ws.p), need, b, di, dout, p, dt, nullptr);
      if (want_dx) write_file(argv[10], dx);
      write_file(argv[11], dc);
    }
  } else if (op == "circ_step" && argc == 13) {
    const int64_t b = arg(argv, 2), di = arg(argv, 3), dout = arg(argv, 4), p = arg(argv, 5);
    const int dt = static_cast<int>(arg(argv, 6));
    Buf x = read_file(argv[7], b * di * esize(dt));
    Buf c = read_file(argv[8], (dout / p) * di * 4);
    Buf dy = read_file(argv[9], b * dout * esize(dt));
    const bool want_dx = std::strcmp(argv[11], "-") != 0;
    Buf y = alloc(b * dout * esize(dt));
    Buf dx = alloc(b * di * esize(dt));
    Buf dc = alloc((dout / p) * di * 4);
    for (size_t i = 0; i < dc.n / 4; ++i) static_cast<float*>(dc.p)[i] = 12345.0f;  // cleared by the forward
    st = circulant_fwd_zero(x.p, static_cast<const float*>(c.p), y.p, static_cast<float*>(dc.p), b, di, dout, p, dt,
                            nullptr);
    for (int rep = 0; rep < 2 && st == RDFFT_OK; ++rep)
      st = circulant_bwd_acc(x.p, static_cast<const float*>(c.p), dy.p, want_dx ? dx.p : nullptr,
                             static_cast<float*>(dc.p), b, di, dout, p, dt, nullptr);
    write_file(argv[10], y);
    if (want_dx) write_file(argv[11], dx);
    write_file(argv[12], dc);
  } else if (op == "circ_spec" && argc == 15) {
    const int64_t b = arg(argv, 2), di = arg(argv, 3), dout = arg(argv, 4), p = arg(argv, 5);
    const int dt = static_cast<int>(arg(argv, 6));
    Buf x = read_file(argv[7], b * di * esize(dt));
    Buf c = read_file(argv[8], (dout / p) * di * 4);
    Buf dy = read_file(argv[9], b * dout * esize(dt));
    const bool want_dx = std::strcmp(argv[12], "-") != 0;
    Buf cs = alloc((dout / p) * di * 4), cs2 = alloc((dout / p) * di * 4);
    Buf y = alloc(b * dout * esize(dt)), y2 = alloc(b * dout * esize(dt));
    Buf dx = alloc(b * di * esize(dt));
    Buf dc = alloc((dout / p) * di * 4);
    for (size_t i = 0; i < cs.n / 4; ++i) static_cast<float*>(cs.p)[i] = static_cast<float*>(cs2.p)[i] = -555.0f;
    for (size_t i = 0; i < dc.n / 4; ++i) static_cast<float*>(dc.p)[i] = 12345.0f;  // cleared by the forward
    auto* pcs = static_cast<float*>(cs.p);
    st = circulant_fwd_step(x.p, static_cast<const float*>(c.p), y.p, static_cast<float*>(dc.p), pcs, b, di, dout, p, dt,
                            nullptr);
    if (st == RDFFT_OK)
      st = circulant_weight_spectra(static_cast<const float*>(c.p), static_cast<float*>(cs2.p), di, dout, p, nullptr);
    if (st == RDFFT_OK && std::memcmp(cs.p, cs2.p, cs.n) != 0) {
      std::fprintf(stderr, "circulant_fwd_step and circulant_weight_spectra wrote different spectra\n");
      return 3;
    }
    if (st == RDFFT_OK) st = circulant_fwd_spec(x.p, pcs, y2.p, nullptr, b, di, dout, p, dt, nullptr);
    for (int rep = 0; rep < 2 && st == RDFFT_OK; ++rep)
      st = circulant_bwd_spec(x.p, pcs, dy.p, want_dx ? dx.p : nullptr, static_cast<float*>(dc.p), rep, b, di, dout, p,
                              dt, nullptr);
    write_file(argv[10], y);
    write_file(argv[11], y2);
    if (want_dx) write_file(argv[12], dx);
    write_file(argv[13], dc);
    write_file(argv[14], cs);
  } else if (op == "cases" && argc == 2) {
    char buf[4096];
    while (std::fgets(buf, sizeof(buf), stdin)) {
      std::string line(buf);
      while (!line.empty() && (line.back() == '\n' || line.back() == '\r')) line.pop_back();
      if (!line.empty()) std::printf("%d\n", call_case(line));
    }
    st = 0;
  } else if (op == "selftest" && argc == 3) {
    Buf out = alloc(64 * 4);
    hipLaunchKernelGGL((selftest_kernel), dim3(1), dim3(64), 0, nullptr, static_cast<float*>(out.p),
                       std::strcmp(argv[2], "ok") == 0 ? 1 : 0);
    st = 0;
  } else {
    std::fprintf(stderr, "bad arguments\n");
    return 2;
  }
  std::printf("status %d launches %ld workgroups %ld\n", st, emu::launches, emu::workgroups);
  return 0;
}
