// Host half of libkvevict: error plumbing, the calibration-artifact reader and
// writer, the filter estimators and byte accounting.  Nothing here touches the
// GPU; these run once per model or once per stream, off the eviction hot path.
#include <math.h>

#include <cmath>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <array>
#include <exception>
#include <mutex>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "kvevict.h"
#include "kvx_common.h"

namespace kvx {

static thread_local std::string g_error;

int set_error(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return code;
}

void clear_error() { g_error.clear(); }

namespace {

// ---------------------------------------------------------------------------
// Symmetric eigen-decomposition by cyclic Jacobi rotations (fp64).  Each
// rotation zeroes one off-diagonal pair; sweeps repeat until the off-diagonal
// mass is negligible against the matrix norm.  Returns the eigenvalues in
// `lam` and the eigenvectors as the columns of `V` (row-major n x n).
// ---------------------------------------------------------------------------
void jacobi_eigen(std::vector<double> &A, int n, std::vector<double> &lam, std::vector<double> &V) {
    V.assign((size_t)n * n, 0.0);
    for (int i = 0; i < n; ++i) V[(size_t)i * n + i] = 1.0;
    double frob = 0.0;
    for (double a : A) frob += a * a;
    for (int sweep = 0; sweep < 60; ++sweep) {
        double off = 0.0;
        for (int p = 0; p < n; ++p)
            for (int q = p + 1; q < n; ++q) off += A[(size_t)p * n + q] * A[(size_t)p * n + q];
        if (off <= 1e-32 * frob) break;
        for (int p = 0; p < n - 1; ++p) {
            for (int q = p + 1; q < n; ++q) {
                const double apq = A[(size_t)p * n + q];
                if (apq == 0.0) continue;
                const double app = A[(size_t)p * n + p], aqq = A[(size_t)q * n + q];
                // rotation angle: tan(theta) = t solves t^2 + 2 t zeta - 1 = 0, smaller root
                const double zeta = (aqq - app) / (2.0 * apq);
                const double t = (zeta >= 0.0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
                const double c = 1.0 / sqrt(1.0 + t * t), s = t * c;
                for (int k = 0; k < n; ++k) {  // columns p, q
                    const double akp = A[(size_t)k * n + p], akq = A[(size_t)k * n + q];
                    A[(size_t)k * n + p] = c * akp - s * akq;
                    A[(size_t)k * n + q] = s * akp + c * akq;
                }
                for (int k = 0; k < n; ++k) {  // rows p, q
                    const double apk = A[(size_t)p * n + k], aqk = A[(size_t)q * n + k];
                    A[(size_t)p * n + k] = c * apk - s * aqk;
                    A[(size_t)q * n + k] = s * apk + c * aqk;
                }
                A[(size_t)p * n + q] = A[(size_t)q * n + p] = 0.0;
                for (int k = 0; k < n; ++k) {
                    const double vkp = V[(size_t)k * n + p], vkq = V[(size_t)k * n + q];
                    V[(size_t)k * n + p] = c * vkp - s * vkq;
                    V[(size_t)k * n + q] = s * vkp + c * vkq;
                }
            }
        }
    }
    lam.resize(n);
    for (int i = 0; i < n; ++i) lam[i] = A[(size_t)i * n + i];
}

// Top eigenvector of the Gram matrix X^T X of X [m, n] (fp64).  Fails when the
// top two singular values of X are not separated (sigma1 - sigma2 <= 1e-12
// sigma1) or X is zero.
int top_right_singular(const std::vector<double> &X, int64_t m, int n, std::vector<double> &v1,
                       const char **why) {
    std::vector<double> Gm((size_t)n * n, 0.0);
    for (int64_t r = 0; r < m; ++r) {
        const double *x = &X[(size_t)r * n];
        for (int i = 0; i < n; ++i) {
            const double xi = x[i];
            if (xi == 0.0) continue;
            double *g = &Gm[(size_t)i * n];
            for (int j = i; j < n; ++j) g[j] += xi * x[j];
        }
    }
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < i; ++j) Gm[(size_t)i * n + j] = Gm[(size_t)j * n + i];
    std::vector<double> lam, V;
    jacobi_eigen(Gm, n, lam, V);
    int i1 = 0;
    for (int i = 1; i < n; ++i)
        if (lam[i] > lam[i1]) i1 = i;
    double l2 = 0.0;
    for (int i = 0; i < n; ++i)
        if (i != i1) l2 = std::max(l2, lam[i]);
    const double s1 = sqrt(std::max(lam[i1], 0.0)), s2 = sqrt(std::max(l2, 0.0));
    if (!(s1 > 0.0)) {
        *why = "the matrix is zero";
        return KVX_EINVAL;
    }
    if (s1 - s2 <= 1e-12 * s1) {
        *why = "the top two singular values coincide";
        return KVX_EINVAL;
    }
    v1.resize(n);
    double nrm = 0.0;
    for (int i = 0; i < n; ++i) {
        v1[i] = V[(size_t)i * n + i1];
        nrm += v1[i] * v1[i];
    }
    nrm = sqrt(nrm);
    for (int i = 0; i < n; ++i) v1[i] /= nrm;
    return KVX_OK;
}

// IEEE binary16 bits to double (exact; subnormals, infinities and NaN kept).
double half_to_double(uint16_t h) {
    const int sign = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
    double v;
    if (e == 0)
        v = std::ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = std::ldexp((double)(m | 0x400), e - 25);
    return sign ? -v : v;
}

// Element i of a K/V row buffer of the given type, widened to double.
double widen_elem(const void *k, int32_t dtype, int64_t i) {
    if (dtype == KVX_F32) return ((const float *)k)[i];
    const uint16_t b = ((const uint16_t *)k)[i];
    if (dtype == KVX_F16) return half_to_double(b);
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

// Runs fn(i) for i in [0, n) on up to 16 worker threads.  An exception in a
// worker (or in starting one) is rethrown here once every started worker
// has been joined.
template <class F>
void parallel_for(int64_t n, F fn) {
    const int64_t hw = std::max(1u, std::thread::hardware_concurrency());
    const int64_t nt = std::min<int64_t>(std::min<int64_t>(hw, 16), n);
    if (nt <= 1) {
        for (int64_t i = 0; i < n; ++i) fn(i);
        return;
    }
    std::exception_ptr err;
    std::mutex mu;
    auto work = [&](int64_t w) {
        try {
            for (int64_t i = w; i < n; i += nt) fn(i);
        } catch (...) {
            std::lock_guard<std::mutex> lock(mu);
            if (!err) err = std::current_exception();
        }
    };
    std::vector<std::thread> th;
    try {
        for (int64_t w = 0; w < nt; ++w) th.emplace_back(work, w);
    } catch (...) {
        for (auto &x : th) x.join();
        throw;
    }
    for (auto &x : th) x.join();
    if (err) std::rethrow_exception(err);
}

// Runs an entry point's body so that no C++ exception crosses the C ABI: host
// memory that cannot be had is KVX_ERANGE, anything else the entry point's
// `code`, each with a message in kvx_last_error().
template <class F>
int guarded(const char *what, int code, F &&body) {
    try {
        return body();
    } catch (const std::bad_alloc &) {
        return set_error(KVX_ERANGE, "%s: out of host memory", what);
    } catch (const std::exception &e) {
        return set_error(code, "%s: %s", what, e.what());
    } catch (...) {
        return set_error(code, "%s: unexpected failure", what);
    }
}

// ---------------------------------------------------------------------------
// .npz artifact: a ZIP archive of "stored" (uncompressed) .npy members.
// ---------------------------------------------------------------------------
uint32_t rd32(const unsigned char *p) { return p[0] | (p[1] << 8) | (p[2] << 16) | ((uint32_t)p[3] << 24); }
uint16_t rd16(const unsigned char *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
uint64_t rd64(const unsigned char *p) { return rd32(p) | ((uint64_t)rd32(p + 4) << 32); }

struct NpyArray {
    std::string descr;
    bool fortran = false;
    std::vector<int64_t> shape;
    std::string data;  // raw element bytes
};

bool parse_npy(const std::string &blob, NpyArray *a) {
    if (blob.size() < 10 || memcmp(blob.data(), "\x93NUMPY", 6) != 0) return false;
    const unsigned char *p = (const unsigned char *)blob.data();
    const int major = p[6];
    size_t hlen, hoff;
    if (major == 1) {
        hlen = rd16(p + 8);
        hoff = 10;
    } else if (major == 2 || major == 3) {
        if (blob.size() < 12) return false;
        hlen = rd32(p + 8);
        hoff = 12;
    } else {
        return false;
    }
    if (hoff + hlen > blob.size()) return false;
    const std::string h = blob.substr(hoff, hlen);
    auto field = [&](const char *name) -> size_t {
        const size_t k = h.find(std::string("'") + name + "'");
        return k == std::string::npos ? k : h.find(':', k);
    };
    size_t k = field("descr");
    if (k == std::string::npos) return false;
    size_t q1 = h.find('\'', k), q2 = q1 == std::string::npos ? q1 : h.find('\'', q1 + 1);
    if (q2 == std::string::npos) return false;
    a->descr = h.substr(q1 + 1, q2 - q1 - 1);
    k = field("fortran_order");
    if (k == std::string::npos) return false;
    const size_t fv = h.find_first_not_of(" :", k);
    if (fv == std::string::npos) return false;  // the header ends before the value
    a->fortran = h.compare(fv, 4, "True") == 0;
    k = field("shape");
    if (k == std::string::npos) return false;
    const size_t o = h.find('(', k), c = h.find(')', k);
    if (o == std::string::npos || c == std::string::npos || c < o) return false;
    a->shape.clear();
    std::string dims = h.substr(o + 1, c - o - 1);
    size_t pos = 0;
    while (pos < dims.size()) {
        const size_t e = dims.find(',', pos);
        std::string tok = dims.substr(pos, e == std::string::npos ? std::string::npos : e - pos);
        tok.erase(0, tok.find_first_not_of(' '));
        if (!tok.empty()) a->shape.push_back(strtoll(tok.c_str(), nullptr, 10));
        if (e == std::string::npos) break;
        pos = e + 1;
    }
    a->data = blob.substr(hoff + hlen);
    return true;
}

// CRC-32 of the ZIP format (reflected polynomial 0xEDB88320).  The table is a
// function-local static, so its one-time initialisation is thread-safe.
uint32_t crc32_of(const unsigned char *d, size_t n) {
    static const std::array<uint32_t, 256> table = [] {
        std::array<uint32_t, 256> t{};
        for (uint32_t i = 0; i < 256; ++i) {
            uint32_t c = i;
            for (int k = 0; k < 8; ++k) c = (c & 1) ? 0xEDB88320u ^ (c >> 1) : c >> 1;
            t[i] = c;
        }
        return t;
    }();
    uint32_t c = 0xFFFFFFFFu;
    for (size_t i = 0; i < n; ++i) c = table[(c ^ d[i]) & 0xFF] ^ (c >> 8);
    return c ^ 0xFFFFFFFFu;
}
uint32_t crc32_of(const std::string &d) { return crc32_of((const unsigned char *)d.data(), d.size()); }

// Whether [off, off + len) lies inside a buffer of `size` bytes (no overflow).
inline bool in_file(uint64_t off, uint64_t len, uint64_t size) { return off <= size && len <= size - off; }

// Reads every stored member of a ZIP archive through its central directory,
// checking each member's CRC-32.
int read_zip(const char *path, std::vector<std::pair<std::string, std::string>> *members) {
    FILE *f = fopen(path, "rb");
    if (!f) return set_error(KVX_EIO, "cannot open '%s'", path);
    std::string buf;
    char chunk[1 << 16];
    size_t n;
    while ((n = fread(chunk, 1, sizeof chunk, f)) > 0) buf.append(chunk, n);
    fclose(f);
    const unsigned char *b = (const unsigned char *)buf.data();
    const size_t size = buf.size();
    if (size < 22) return set_error(KVX_EIO, "'%s' is not a zip archive", path);
    size_t eocd = std::string::npos;
    for (size_t i = size - 22 + 1; i-- > 0 && size - i <= 22 + 65535;)
        if (rd32(b + i) == 0x06054b50u) {
            eocd = i;
            break;
        }
    if (eocd == std::string::npos) return set_error(KVX_EIO, "'%s': no zip end record", path);
    uint64_t count = rd16(b + eocd + 10);
    uint64_t cd_off = rd32(b + eocd + 16);
    if (cd_off == 0xFFFFFFFFu || count == 0xFFFFu) {  // ZIP64 end record via its locator
        if (eocd < 20 || rd32(b + eocd - 20) != 0x07064b50u) return set_error(KVX_EIO, "'%s': bad zip64 locator", path);
        const uint64_t z = rd64(b + eocd - 20 + 8);
        if (!in_file(z, 56, size) || rd32(b + z) != 0x06064b50u)
            return set_error(KVX_EIO, "'%s': bad zip64 end record", path);
        count = rd64(b + z + 32);
        cd_off = rd64(b + z + 48);
    }
    size_t p = cd_off;
    for (uint64_t e = 0; e < count; ++e) {
        if (!in_file(p, 46, size) || rd32(b + p) != 0x02014b50u)
            return set_error(KVX_EIO, "'%s': bad central directory", path);
        const uint16_t method = rd16(b + p + 10);
        const uint32_t crc = rd32(b + p + 16);
        uint64_t csize = rd32(b + p + 20), usize = rd32(b + p + 24);
        const uint16_t nlen = rd16(b + p + 28), xlen = rd16(b + p + 30), clen = rd16(b + p + 32);
        uint64_t lho = rd32(b + p + 42);
        if (!in_file(p + 46, (uint64_t)nlen + xlen, size)) return set_error(KVX_EIO, "'%s': truncated entry", path);
        std::string name((const char *)b + p + 46, nlen);
        const unsigned char *x = b + p + 46 + nlen, *xe = x + xlen;
        while (xe - x >= 4) {  // ZIP64 extra: the fields that overflowed, in this order
            const uint16_t id = rd16(x), sz = rd16(x + 2);
            if (sz > xe - x - 4) break;  // a field running past the extra block
            const unsigned char *d = x + 4, *fe = x + 4 + sz;
            if (id == 0x0001) {
                if (usize == 0xFFFFFFFFu && fe - d >= 8) usize = rd64(d), d += 8;
                if (csize == 0xFFFFFFFFu && fe - d >= 8) csize = rd64(d), d += 8;
                if (lho == 0xFFFFFFFFu && fe - d >= 8) lho = rd64(d), d += 8;
            }
            x = fe;
        }
        if (method != 0) return set_error(KVX_EIO, "'%s': member '%s' is compressed (only stored members are read)", path, name.c_str());
        if (csize != usize) return set_error(KVX_EIO, "'%s': member '%s' has inconsistent sizes", path, name.c_str());
        if (!in_file(lho, 30, size) || rd32(b + lho) != 0x04034b50u)
            return set_error(KVX_EIO, "'%s': bad local header", path);
        const uint64_t data = lho + 30 + rd16(b + lho + 26) + rd16(b + lho + 28);
        if (!in_file(data, csize, size)) return set_error(KVX_EIO, "'%s': member '%s' is truncated", path, name.c_str());
        if (crc32_of(b + data, csize) != crc)
            return set_error(KVX_EIO, "'%s': member '%s' fails its CRC-32 check", path, name.c_str());
        members->emplace_back(name, buf.substr(data, csize));
        p += 46 + nlen + xlen + clen;
    }
    return KVX_OK;
}

// UTF-32LE ('<U' numpy strings) to UTF-8.
std::string utf32_to_utf8(const std::string &raw) {
    std::string s;
    for (size_t i = 0; i + 4 <= raw.size(); i += 4) {
        const uint32_t c = rd32((const unsigned char *)raw.data() + i);
        if (c == 0) break;
        if (c < 0x80) {
            s += (char)c;
        } else if (c < 0x800) {
            s += (char)(0xC0 | (c >> 6));
            s += (char)(0x80 | (c & 0x3F));
        } else if (c < 0x10000) {
            s += (char)(0xE0 | (c >> 12));
            s += (char)(0x80 | ((c >> 6) & 0x3F));
            s += (char)(0x80 | (c & 0x3F));
        } else {
            s += (char)(0xF0 | (c >> 18));
            s += (char)(0x80 | ((c >> 12) & 0x3F));
            s += (char)(0x80 | ((c >> 6) & 0x3F));
            s += (char)(0x80 | (c & 0x3F));
        }
    }
    return s;
}

std::vector<uint32_t> utf8_to_utf32(const char *s) {
    std::vector<uint32_t> out;
    const unsigned char *p = (const unsigned char *)s;
    while (*p) {
        uint32_t c = *p++;
        int extra = c >= 0xF0 ? 3 : c >= 0xE0 ? 2 : c >= 0xC0 ? 1 : 0;
        c &= extra == 3 ? 0x07 : extra == 2 ? 0x0F : extra == 1 ? 0x1F : 0x7F;
        while (extra-- > 0 && (*p & 0xC0) == 0x80) c = (c << 6) | (*p++ & 0x3F);
        out.push_back(c);
    }
    return out;
}

bool npy_string(const NpyArray &a, std::string *out) {
    if (a.descr.size() < 3 || a.descr.compare(0, 2, "<U") != 0 || !a.shape.empty()) return false;
    *out = utf32_to_utf8(a.data);
    return true;
}

bool npy_int64(const NpyArray &a, int64_t *out) {
    if (!a.shape.empty() || a.data.size() < 8) return false;
    if (a.descr == "<i8") {
        memcpy(out, a.data.data(), 8);
        return true;
    }
    return false;
}



std::string npy_blob(const std::string &descr, const std::vector<int64_t> &shape, const std::string &data) {
    std::string shp = "(";
    for (size_t i = 0; i < shape.size(); ++i) shp += std::to_string(shape[i]) + (shape.size() == 1 ? ",)" : i + 1 < shape.size() ? ", " : ")");
    if (shape.empty()) shp += ")";
    std::string h = "{'descr': '" + descr + "', 'fortran_order': False, 'shape': " + shp + ", }";
    const size_t total = 10 + h.size() + 1;
    h.append((64 - total % 64) % 64, ' ');
    h += '\n';
    std::string out("\x93NUMPY\x01\x00", 8);
    out += (char)(h.size() & 0xFF);
    out += (char)(h.size() >> 8);
    return out + h + data;
}

void put16(std::string &s, uint32_t v) {
    s += (char)(v & 0xFF);
    s += (char)((v >> 8) & 0xFF);
}
void put32(std::string &s, uint32_t v) {
    put16(s, v & 0xFFFF);
    put16(s, v >> 16);
}

std::string utf32_bytes(const char *s) {
    std::string raw;
    for (uint32_t c : utf8_to_utf32(s)) put32(raw, c);
    return raw;
}

}  // namespace
}  // namespace kvx

using namespace kvx;

extern "C" {

KVX_API const char *kvx_last_error(void) { return g_error.c_str(); }

KVX_API int kvx_abi_version(void) { return 1; }

static int qf_filters_load_body(const char *path, const char *expect_model_id, int64_t L, int64_t H_kv, int64_t D,
                                float *out, int64_t *n_samples_out) {
    clear_error();
    if (!path || !out || L <= 0 || H_kv <= 0 || D <= 0)
        return set_error(KVX_EINVAL, "qf_filters_load: bad arguments");
    std::vector<std::pair<std::string, std::string>> members;
    int rc = read_zip(path, &members);
    if (rc) return rc;
    auto get = [&](const char *name, NpyArray *a) -> int {
        const std::string want = std::string(name) + ".npy";
        for (auto &m : members)
            if (m.first == want) {
                if (!parse_npy(m.second, a)) return set_error(KVX_EIO, "'%s': field '%s' is not a valid .npy", path, name);
                return KVX_OK;
            }
        return set_error(KVX_EIO, "'%s': field '%s' is missing", path, name);
    };
    NpyArray fa, ma, va, na, da;
    if ((rc = get("filters", &fa)) || (rc = get("model_id", &ma)) || (rc = get("version", &va)) ||
        (rc = get("n_samples", &na)) || (rc = get("dataset", &da)))
        return rc;
    int64_t version = 0, n_samples = 0;
    std::string model_id, dataset;
    if (!npy_int64(va, &version) || !npy_int64(na, &n_samples))
        return set_error(KVX_EIO, "'%s': version and n_samples must be int64 scalars", path);
    if (!npy_string(ma, &model_id) || !npy_string(da, &dataset))
        return set_error(KVX_EIO, "'%s': model_id and dataset must be string scalars", path);
    if (version != 1)
        return set_error(KVX_EMISMATCH, "'%s': artifact version %lld is not supported (expected 1)", path, (long long)version);
    if (expect_model_id && model_id != expect_model_id)
        return set_error(KVX_EMISMATCH, "'%s': filters were calibrated for '%s', not '%s'", path, model_id.c_str(),
                         expect_model_id);
    if (fa.descr != "<f4" || fa.fortran) return set_error(KVX_EIO, "'%s': filters must be little-endian float32, C order", path);
    if (fa.shape.size() != 3) return set_error(KVX_EMISMATCH, "'%s': filters must be [layers, kv_heads, head_dim]", path);
    if (fa.shape[0] != L)
        return set_error(KVX_EMISMATCH, "'%s': artifact has %lld layers, the model has %lld (missing layer)", path,
                         (long long)fa.shape[0], (long long)L);
    if (fa.shape[1] != H_kv || fa.shape[2] != D)
        return set_error(KVX_EMISMATCH, "'%s': head layout [%lld, %lld] differs from the model's [%lld, %lld]", path,
                         (long long)fa.shape[1], (long long)fa.shape[2], (long long)H_kv, (long long)D);
    const size_t bytes = (size_t)(L * H_kv * D) * 4;
    if (fa.data.size() < bytes) return set_error(KVX_EIO, "'%s': filters data is truncated", path);
    memcpy(out, fa.data.data(), bytes);
    if (n_samples_out) *n_samples_out = n_samples;
    return KVX_OK;
}

static int qf_filters_save_body(const char *path, const float *filters, int64_t L, int64_t H_kv, int64_t D,
                                const char *model_id, int64_t n_samples, const char *dataset) {
    clear_error();
    if (!path || !filters || !model_id || !dataset || L <= 0 || H_kv <= 0 || D <= 0)
        return set_error(KVX_EINVAL, "qf_filters_save: bad arguments");
    struct Member {
        std::string name, blob;
    };
    std::vector<Member> ms;
    const std::string fdata((const char *)filters, (size_t)(L * H_kv * D) * 4);
    ms.push_back({"filters.npy", npy_blob("<f4", {L, H_kv, D}, fdata)});
    const std::string mid = utf32_bytes(model_id), ds = utf32_bytes(dataset);
    ms.push_back({"model_id.npy", npy_blob("<U" + std::to_string(std::max<size_t>(1, mid.size() / 4)), {},
                                           mid.empty() ? std::string(4, '\0') : mid)});
    std::string v(8, '\0'), ns(8, '\0');
    const int64_t one = 1;
    memcpy(&v[0], &one, 8);
    memcpy(&ns[0], &n_samples, 8);
    ms.push_back({"version.npy", npy_blob("<i8", {}, v)});
    ms.push_back({"n_samples.npy", npy_blob("<i8", {}, ns)});
    ms.push_back({"dataset.npy", npy_blob("<U" + std::to_string(std::max<size_t>(1, ds.size() / 4)), {},
                                          ds.empty() ? std::string(4, '\0') : ds)});
    std::string zip, cd;
    for (auto &m : ms) {
        const uint32_t crc = crc32_of(m.blob), off = (uint32_t)zip.size(), sz = (uint32_t)m.blob.size();
        if ((uint64_t)zip.size() + m.blob.size() > 0xFFFFFFF0ull)
            return set_error(KVX_EINVAL, "qf_filters_save: artifact larger than 4 GiB");
        put32(zip, 0x04034b50u); put16(zip, 20); put16(zip, 0); put16(zip, 0); put16(zip, 0); put16(zip, 0x21);
        put32(zip, crc); put32(zip, sz); put32(zip, sz); put16(zip, (uint32_t)m.name.size()); put16(zip, 0);
        zip += m.name;
        zip += m.blob;
        put32(cd, 0x02014b50u); put16(cd, 20); put16(cd, 20); put16(cd, 0); put16(cd, 0); put16(cd, 0);
        put16(cd, 0x21); put32(cd, crc); put32(cd, sz); put32(cd, sz); put16(cd, (uint32_t)m.name.size());
        put16(cd, 0); put16(cd, 0); put16(cd, 0); put16(cd, 0); put32(cd, 0); put32(cd, off);
        cd += m.name;
    }
    const uint32_t cd_off = (uint32_t)zip.size();
    zip += cd;
    put32(zip, 0x06054b50u); put16(zip, 0); put16(zip, 0); put16(zip, (uint32_t)ms.size());
    put16(zip, (uint32_t)ms.size()); put32(zip, (uint32_t)cd.size()); put32(zip, cd_off); put16(zip, 0);
    FILE *f = fopen(path, "wb");
    if (!f) return set_error(KVX_EIO, "cannot create '%s'", path);
    const bool ok = fwrite(zip.data(), 1, zip.size(), f) == zip.size();
    if (fclose(f) != 0 || !ok) return set_error(KVX_EIO, "short write to '%s'", path);
    return KVX_OK;
}

static int qf_filters_from_queries_body(const float *q, int64_t H_q, int64_t N, int64_t D, int64_t H_kv, float *out) {
    clear_error();
    if (!q || !out || H_q <= 0 || N <= 0 || D <= 0 || D > 4096 || H_kv <= 0)
        return set_error(KVX_EINVAL, "qf_filters_from_queries: bad arguments");
    if (H_q % H_kv) return set_error(KVX_EINVAL, "qf_filters_from_queries: H_q (%lld) must be a multiple of H_kv (%lld)",
                                     (long long)H_q, (long long)H_kv);
    const int n = (int)D;
    std::vector<std::vector<double>> f((size_t)H_q);
    std::vector<int> status((size_t)H_q, KVX_OK);
    std::vector<const char *> why((size_t)H_q, "");
    parallel_for(H_q, [&](int64_t h) {
        std::vector<double> X((size_t)(N * D));
        const float *src = q + (size_t)h * N * D;
        for (int64_t i = 0; i < N * D; ++i) {
            if (!std::isfinite(src[i])) {
                status[h] = KVX_EINVAL;
                why[h] = "non-finite activation";
                return;
            }
            X[i] = src[i];
        }
        std::vector<double> v1;
        status[h] = top_right_singular(X, N, n, v1, &why[h]);
        if (status[h]) return;
        // sign of 1^T u1 = sign of sum_r (x_r . v1); a zero sum counts as +
        double proj = 0.0;
        for (int64_t r = 0; r < N; ++r) {
            double d = 0.0;
            for (int i = 0; i < n; ++i) d += X[(size_t)r * n + i] * v1[i];
            proj += d;
        }
        if (proj < 0.0)
            for (double &x : v1) x = -x;
        f[h] = v1;
    });
    for (int64_t h = 0; h < H_q; ++h)
        if (status[h]) return set_error(status[h], "qf_filters_from_queries: head %lld: %s", (long long)h, why[h]);
    const int64_t grp = H_q / H_kv;
    for (int64_t j = 0; j < H_kv; ++j) {
        std::vector<double> m((size_t)n, 0.0);
        for (int64_t h = j * grp; h < (j + 1) * grp; ++h)
            for (int i = 0; i < n; ++i) m[i] += f[h][i];
        double nrm = 0.0;
        for (int i = 0; i < n; ++i) {
            m[i] /= (double)grp;
            nrm += m[i] * m[i];
        }
        nrm = sqrt(nrm);
        if (!(nrm > 0.0)) return set_error(KVX_EINVAL, "qf_filters_from_queries: KV head %lld: zero group mean", (long long)j);
        for (int i = 0; i < n; ++i) out[(size_t)j * n + i] = (float)(m[i] / nrm);
    }
    return KVX_OK;
}

static int qf_filters_from_keys_body(const void *k, int32_t dtype, int64_t G, int64_t n, int64_t group_stride,
                                     int64_t D, float *out) {
    clear_error();
    if (!k || !out || G < 0 || n <= 1 || D <= 0 || D > 4096 || group_stride < n)
        return set_error(KVX_EINVAL, "qf_filters_from_keys: bad arguments");
    if (dtype != KVX_BF16 && dtype != KVX_F32 && dtype != KVX_F16)
        return set_error(KVX_EINVAL, "qf_filters_from_keys: bad dtype");
    const int dd = (int)D;
    std::vector<int> status((size_t)G, KVX_OK);
    std::vector<const char *> why((size_t)G, "");
    parallel_for(G, [&](int64_t g) {
        std::vector<double> X((size_t)(n * D));
        for (int64_t r = 0; r < n; ++r)
            for (int i = 0; i < dd; ++i) {
                const double x = widen_elem(k, dtype, (g * group_stride + r) * D + i);
                if (!std::isfinite(x)) {
                    status[g] = KVX_EINVAL;
                    why[g] = "non-finite key";
                    return;
                }
                X[(size_t)r * dd + i] = x;
            }
        for (int i = 0; i < dd; ++i) {  // subtract the column means
            double mean = 0.0;
            for (int64_t r = 0; r < n; ++r) mean += X[(size_t)r * dd + i];
            mean /= (double)n;
            for (int64_t r = 0; r < n; ++r) X[(size_t)r * dd + i] -= mean;
        }
        std::vector<double> v1;
        status[g] = top_right_singular(X, n, dd, v1, &why[g]);
        if (status[g]) return;
        int imax = 0;
        for (int i = 1; i < dd; ++i)
            if (fabs(v1[i]) > fabs(v1[imax])) imax = i;
        const double sg = v1[imax] > 0.0 ? 1.0 : -1.0;
        for (int i = 0; i < dd; ++i) out[(size_t)g * dd + i] = (float)(sg * v1[i]);
    });
    for (int64_t g = 0; g < G; ++g)
        if (status[g]) return set_error(status[g], "qf_filters_from_keys: group %lld: %s", (long long)g, why[g]);
    return KVX_OK;
}

KVX_API int kvx_stats(kvx_shape shape, int64_t tokens_seen, int64_t tokens_kept, int32_t mode, kvx_stats_t *out) {
    clear_error();
    if (!out || shape.L < 0 || shape.B < 0 || shape.H < 0 || shape.D <= 0 || tokens_seen < 0 || tokens_kept < 0 ||
        tokens_kept > tokens_seen || (shape.dtype != KVX_BF16 && shape.dtype != KVX_F32 && shape.dtype != KVX_F16))
        return set_error(KVX_EINVAL, "kvx_stats: bad arguments");
    const int64_t G = shape.L * shape.B * shape.H, es = shape.dtype == KVX_F32 ? 4 : 2;
    out->tokens_seen = tokens_seen;
    out->tokens_kept = tokens_kept;
    out->kept_bytes = G * tokens_kept * 2 * shape.D * es;
    out->full_seq_bytes = G * tokens_seen * 2 * shape.D * es;
    out->compression_ratio = out->kept_bytes ? (double)out->full_seq_bytes / (double)out->kept_bytes : 0.0;
    out->filter_bytes = mode == KVX_SCORE_PROJ ? shape.L * shape.H * shape.D * 4 : 0;
    return KVX_OK;
}

// The four host entry points that parse files or allocate host memory, each
// run through guarded() so that a failure is a status, never an exception.
KVX_API int qf_filters_load(const char *path, const char *expect_model_id, int64_t L, int64_t H_kv, int64_t D,
                            float *out, int64_t *n_samples_out) {
    return guarded("qf_filters_load", KVX_EIO, [&] {
        return qf_filters_load_body(path, expect_model_id, L, H_kv, D, out, n_samples_out);
    });
}

KVX_API int qf_filters_save(const char *path, const float *filters, int64_t L, int64_t H_kv, int64_t D,
                            const char *model_id, int64_t n_samples, const char *dataset) {
    return guarded("qf_filters_save", KVX_EIO, [&] {
        return qf_filters_save_body(path, filters, L, H_kv, D, model_id, n_samples, dataset);
    });
}

KVX_API int qf_filters_from_queries(const float *q, int64_t H_q, int64_t N, int64_t D, int64_t H_kv, float *out) {
    return guarded("qf_filters_from_queries", KVX_EINVAL,
                   [&] { return qf_filters_from_queries_body(q, H_q, N, D, H_kv, out); });
}

KVX_API int qf_filters_from_keys(const void *k, int32_t dtype, int64_t G, int64_t n, int64_t group_stride, int64_t D,
                                 float *out) {
    return guarded("qf_filters_from_keys", KVX_EINVAL,
                   [&] { return qf_filters_from_keys_body(k, dtype, G, n, group_stride, D, out); });
}

}  // extern "C"
