// Persisted flat-block files: publish a block stack's extents once to a
// content-addressed directory, then map it read-only as the host backing of
// a store (STAGED, or REGISTER where the platform allows registration).
//
// Design source: "Distributed Layerwise Offload", "Runtime cache" (content
// hashing of tensor names, metadata and final bytes; one content-addressed
// entry per identity; publication into a same-filesystem temporary directory
// that is flushed and atomically renamed; a manifest with SHA-256 digests;
// kernel flock ownership, so a dead writer releases the lock; stale
// temporary entries removed by the next lock owner; a lock wait with a time limit) and
// "Registered runtime-cache transfer" (page-aligned ranges of one mapping).
//
// Entry <dir>/<key>/ holds
//   blocks.bin     block b's extent at offset b * stride, stride = extent
//                  rounded up to 4096 bytes (zero padded), so every extent
//                  starts on a page of the mapping;
//   manifest.json  format, the model descriptor, the tensor table, the
//                  per-block SHA-256 digests and the content digest.
// The content digest (and key, lower-case hex) is SHA-256 over the canonical
// metadata text (see canonical_meta) followed by the 32-byte digests of the
// blocks in order.
#include <fcntl.h>
#include <sys/file.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <sys/types.h>
#include <unistd.h>
#include <dirent.h>

#include <algorithm>
#include <cerrno>
#include <chrono>
#include <cstdio>
#include <cstring>
#include <random>
#include <string>
#include <thread>
#include <vector>

#include "lwo_internal.h"

using namespace lwo;

namespace {

// ------------------------------------------------------------------ SHA-256 (FIPS 180-4)

typedef unsigned __int128 u128;

// floor(n^(1/3)) and floor(n^(1/2)) by bisection (exact integer arithmetic).
uint64_t icbrt(u128 n) {
    uint64_t lo = 0, hi = 1ull << 43;
    while (hi - lo > 1) {
        const uint64_t mid = lo + (hi - lo) / 2;
        if ((u128)mid * mid * mid <= n) lo = mid; else hi = mid;
    }
    return lo;
}
uint64_t isqrt(u128 n) {
    uint64_t lo = 0, hi = 1ull << 63;
    while (hi - lo > 1) {
        const uint64_t mid = lo + (hi - lo) / 2;
        if ((u128)mid * mid <= n) lo = mid; else hi = mid;
    }
    return lo;
}

// Section 4.2.2: K[i] = the first 32 bits of the fractional part of the cube
// root of the i-th prime; section 5.3.3: H0[i] = the same of the square root
// of the first eight primes.  floor(cbrt(p * 2^96)) = floor(cbrt(p) * 2^32),
// whose low 32 bits are those fraction bits (likewise for the square root).
struct ShaConsts {
    uint32_t k[64], h0[8];
    ShaConsts() {
        int found = 0;
        for (uint32_t p = 2; found < 64; ++p) {
            bool prime = true;
            for (uint32_t q = 2; q * q <= p; ++q)
                if (p % q == 0) { prime = false; break; }
            if (!prime) continue;
            k[found] = (uint32_t)icbrt((u128)p << 96);
            if (found < 8) h0[found] = (uint32_t)isqrt((u128)p << 64);
            ++found;
        }
    }
};
const ShaConsts& sha_consts() {
    static const ShaConsts c;
    return c;
}

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

struct Sha256 {
    uint32_t h[8];
    uint8_t buf[64];
    uint64_t total = 0;
    int fill = 0;
    Sha256() { std::memcpy(h, sha_consts().h0, sizeof(h)); }

    void block(const uint8_t* p) {   // section 6.2.2
        const uint32_t* K = sha_consts().k;
        uint32_t w[64];
        for (int t = 0; t < 16; ++t)
            w[t] = (uint32_t)p[4 * t] << 24 | (uint32_t)p[4 * t + 1] << 16 | (uint32_t)p[4 * t + 2] << 8 | p[4 * t + 3];
        for (int t = 16; t < 64; ++t) {
            const uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
            const uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
            w[t] = w[t - 16] + s0 + w[t - 7] + s1;
        }
        uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
        for (int t = 0; t < 64; ++t) {
            const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
            const uint32_t ch = (e & f) ^ (~e & g);
            const uint32_t t1 = hh + S1 + ch + K[t] + w[t];
            const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
            const uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
            const uint32_t t2 = S0 + maj;
            hh = g; g = f; f = e; e = d + t1; d = c; c = b; b = a; a = t1 + t2;
        }
        h[0] += a; h[1] += b; h[2] += c; h[3] += d; h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
    }
    void update(const void* data, uint64_t n) {
        const uint8_t* p = (const uint8_t*)data;
        total += n;
        if (fill) {
            const uint64_t take = std::min<uint64_t>(n, 64 - fill);
            std::memcpy(buf + fill, p, take);
            fill += (int)take; p += take; n -= take;
            if (fill == 64) { block(buf); fill = 0; }
        }
        while (n >= 64) { block(p); p += 64; n -= 64; }
        if (n) { std::memcpy(buf, p, n); fill = (int)n; }
    }
    void final(uint8_t out[32]) {   // section 5.1.1: 1 bit, zeros, 64-bit big-endian bit length
        const uint64_t bits = total * 8;
        const uint8_t one = 0x80, zero = 0;
        update(&one, 1);
        while (fill != 56) update(&zero, 1);
        uint8_t len[8];
        for (int i = 0; i < 8; ++i) len[i] = (uint8_t)(bits >> (56 - 8 * i));
        update(len, 8);
        for (int i = 0; i < 8; ++i)
            for (int j = 0; j < 4; ++j) out[4 * i + j] = (uint8_t)(h[i] >> (24 - 8 * j));
    }
};

std::string hex(const uint8_t* d, int n) {
    static const char* x = "0123456789abcdef";
    std::string s;
    for (int i = 0; i < n; ++i) { s += x[d[i] >> 4]; s += x[d[i] & 15]; }
    return s;
}

bool unhex(const std::string& s, uint8_t* out, int n) {
    if ((int)s.size() != 2 * n) return false;
    auto v = [](char c) { return c >= '0' && c <= '9' ? c - '0' : c >= 'a' && c <= 'f' ? c - 'a' + 10 : -1; };
    for (int i = 0; i < n; ++i) {
        const int a = v(s[2 * i]), b = v(s[2 * i + 1]);
        if (a < 0 || b < 0) return false;
        out[i] = (uint8_t)(a * 16 + b);
    }
    return true;
}

// Per-block digests, blocks spread over up to 16 threads.
void block_digests(const std::vector<const uint8_t*>& ptr, uint64_t bytes, std::vector<uint8_t>& out) {
    const int n = (int)ptr.size();
    out.assign((size_t)n * 32, 0);
    const int nt = (int)std::max(1u, std::min({16u, std::thread::hardware_concurrency(), (unsigned)std::max(n, 1)}));
    std::vector<std::thread> th;
    for (int t = 0; t < nt; ++t)
        th.emplace_back([&, t] {
            for (int b = t; b < n; b += nt) {
                Sha256 h;
                h.update(ptr[b], bytes);
                h.final(&out[(size_t)b * 32]);
            }
        });
    for (auto& x : th) x.join();
}

// ------------------------------------------------------------------ entry metadata

const char* kFormat = "lwo-flat-blocks-2";
constexpr uint64_t kPage = 4096;

// Canonical text of everything that gives the block bytes their meaning.
std::string canonical_meta(const lwo_model_desc& d, const Layout& L) {
    std::string s = std::string(kFormat) + "\n";
    char line[256];
    snprintf(line, sizeof(line), "kind %d n_blocks %d hidden %d heads %d ffn %d act_dtype %d linear_dtype %d extent_bytes %llu\n",
             d.kind, d.n_blocks, d.hidden, d.heads, d.ffn, d.act_dtype, d.linear_dtype,
             (unsigned long long)L.extent_bytes);
    s += line;
    for (const TensorSlot& t : L.tensors) {
        snprintf(line, sizeof(line), "%s %llu %llu %d %d %d %d %s\n", t.name.c_str(), (unsigned long long)t.offset,
                 (unsigned long long)t.bytes, t.dtype, t.rank, t.shape[0], t.shape[1], t.tiled ? "tiled" : "rows");
        s += line;
    }
    return s;
}

void content_digest(const std::string& meta, const std::vector<uint8_t>& digests, uint8_t out[32]) {
    Sha256 h;
    h.update(meta.data(), meta.size());
    h.update(digests.data(), digests.size());
    h.final(out);
}

std::string json_escape(const std::string& s) {
    std::string o;
    for (char c : s) {
        if (c == '"' || c == '\\') { o += '\\'; o += c; }
        else if (c == '\n') o += "\\n";
        else o += c;
    }
    return o;
}

std::string manifest_json(const lwo_model_desc& d, const Layout& L, const std::string& meta, uint64_t stride,
                          const std::vector<uint8_t>& digests, const std::string& key) {
    std::string j = "{\n";
    j += "  \"format\": \"" + std::string(kFormat) + "\",\n";
    j += "  \"key\": \"" + key + "\",\n";
    j += "  \"n_blocks\": " + std::to_string(d.n_blocks) + ",\n";
    j += "  \"extent_bytes\": " + std::to_string(L.extent_bytes) + ",\n";
    j += "  \"stride\": " + std::to_string(stride) + ",\n";
    j += "  \"file\": \"blocks.bin\",\n";
    j += "  \"file_bytes\": " + std::to_string(stride * (uint64_t)d.n_blocks) + ",\n";
    j += "  \"desc\": {\"kind\": " + std::to_string(d.kind) + ", \"n_blocks\": " + std::to_string(d.n_blocks) +
         ", \"hidden\": " + std::to_string(d.hidden) + ", \"heads\": " + std::to_string(d.heads) +
         ", \"ffn\": " + std::to_string(d.ffn) + ", \"act_dtype\": " + std::to_string(d.act_dtype) +
         ", \"linear_dtype\": " + std::to_string(d.linear_dtype) + "},\n";
    j += "  \"tensors\": [\n";
    for (size_t i = 0; i < L.tensors.size(); ++i) {
        const TensorSlot& t = L.tensors[i];
        j += "    {\"name\": \"" + json_escape(t.name) + "\", \"offset\": " + std::to_string(t.offset) +
             ", \"bytes\": " + std::to_string(t.bytes) + ", \"dtype\": " + std::to_string(t.dtype) +
             ", \"tiled\": " + (t.tiled ? "true" : "false") + ", \"shape\": [" +
             std::to_string(t.shape[0]) + (t.rank == 2 ? ", " + std::to_string(t.shape[1]) : std::string()) + "]}" +
             (i + 1 < L.tensors.size() ? ",\n" : "\n");
    }
    j += "  ],\n";
    j += "  \"meta\": \"" + json_escape(meta) + "\",\n";
    j += "  \"block_sha256\": [";
    for (int b = 0; b < d.n_blocks; ++b)
        j += std::string(b ? ", " : "") + "\"" + hex(&digests[(size_t)b * 32], 32) + "\"";
    j += "],\n";
    j += "  \"content_digest\": \"" + key + "\"\n}\n";
    return j;
}

// Minimal readers for the manifest this file writes.
bool json_string(const std::string& j, const std::string& key, std::string& out) {
    const std::string k = "\"" + key + "\": \"";
    size_t p = j.find(k);
    if (p == std::string::npos) return false;
    p += k.size();
    out.clear();
    while (p < j.size() && j[p] != '"') {
        if (j[p] == '\\' && p + 1 < j.size()) {
            ++p;
            out += j[p] == 'n' ? '\n' : j[p];
        } else {
            out += j[p];
        }
        ++p;
    }
    return p < j.size();
}
bool json_u64(const std::string& j, const std::string& key, uint64_t& out) {
    const std::string k = "\"" + key + "\": ";
    size_t p = j.find(k);
    if (p == std::string::npos) return false;
    char* end = nullptr;
    out = std::strtoull(j.c_str() + p + k.size(), &end, 10);
    return end != j.c_str() + p + k.size();
}
bool json_digest_list(const std::string& j, const std::string& key, int n, std::vector<uint8_t>& out) {
    const std::string k = "\"" + key + "\": [";
    size_t p = j.find(k);
    if (p == std::string::npos) return false;
    p += k.size();
    out.assign((size_t)n * 32, 0);
    for (int b = 0; b < n; ++b) {
        const size_t q = j.find('"', p);
        if (q == std::string::npos || q + 65 >= j.size() || j[q + 65] != '"') return false;
        if (!unhex(j.substr(q + 1, 64), &out[(size_t)b * 32], 32)) return false;
        p = q + 66;
    }
    return true;
}

// ------------------------------------------------------------------ files

bool write_all(int fd, const void* data, uint64_t n) {
    const char* p = (const char*)data;
    while (n) {
        const ssize_t w = ::write(fd, p, (size_t)std::min<uint64_t>(n, 1ull << 30));
        if (w <= 0) return false;
        p += w;
        n -= (uint64_t)w;
    }
    return true;
}

bool read_file(const std::string& path, std::string& out) {
    FILE* f = std::fopen(path.c_str(), "rb");
    if (!f) return false;
    out.clear();
    char buf[65536];
    size_t r;
    while ((r = std::fread(buf, 1, sizeof(buf), f)) > 0) out.append(buf, r);
    std::fclose(f);
    return true;
}

bool fsync_path(const std::string& path, int flags) {
    const int fd = ::open(path.c_str(), flags);
    if (fd < 0) return false;
    const bool ok = ::fsync(fd) == 0;
    ::close(fd);
    return ok;
}

void remove_tree(const std::string& path) {
    DIR* d = ::opendir(path.c_str());
    if (d) {
        while (struct dirent* e = ::readdir(d)) {
            const std::string n = e->d_name;
            if (n == "." || n == "..") continue;
            const std::string p = path + "/" + n;
            struct stat st;
            if (::lstat(p.c_str(), &st) == 0 && S_ISDIR(st.st_mode)) remove_tree(p);
            else ::unlink(p.c_str());
        }
        ::closedir(d);
    }
    ::rmdir(path.c_str());
}

bool exists(const std::string& path) {
    struct stat st;
    return ::stat(path.c_str(), &st) == 0;
}

}  // namespace

struct lwo_cache {
    int fd = -1;
    void* base = nullptr;
    uint64_t map_bytes = 0;
    std::vector<const void*> extents;
};

// ------------------------------------------------------------------ C ABI

extern "C" lwo_status lwo_sha256(const void* data, uint64_t bytes, uint8_t* out32) {
    try {
        clear_error();
        if ((!data && bytes) || !out32) { set_error("sha256: NULL argument"); return LWO_EINVAL; }
        Sha256 h;
        h.update(data, bytes);
        h.final(out32);
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_sha256");
    } catch (const std::exception& e) {
        return fail_exception("lwo_sha256", e.what());
    } catch (...) {
        return fail_exception("lwo_sha256", "unknown exception");
    }
}

extern "C" lwo_status lwo_cache_publish(const char* dir, const lwo_model_desc* desc, const lwo_block_source* src,
                                        uint32_t wait_ms, char* key_out, int32_t* created) {
    try {
        clear_error();
        if (!dir || !desc || !src || !key_out || !created) { set_error("cache_publish: NULL argument"); return LWO_EINVAL; }
        if (!src->extents && !src->fill) { set_error("cache_publish: source has neither extents nor fill"); return LWO_EINVAL; }
        LWO_TRY(validate_desc(desc));
        const lwo_model_desc& d = *desc;
        const Layout L = make_layout(d);
        const uint64_t ext = L.extent_bytes, stride = (ext + kPage - 1) / kPage * kPage;
        const int n = d.n_blocks;
        *created = 0;
        key_out[0] = 0;

        // Pass 1: block digests (a fill source is packed into a scratch extent).
        std::vector<uint8_t> digests;
        std::vector<uint8_t> scratch;
        if (src->extents) {
            std::vector<const uint8_t*> ptr(n);
            for (int b = 0; b < n; ++b) {
                if (!src->extents[b]) { set_error("cache_publish: extent " + std::to_string(b) + " is NULL"); return LWO_EINVAL; }
                ptr[b] = (const uint8_t*)src->extents[b];
            }
            block_digests(ptr, ext, digests);
        } else {
            scratch.assign(ext, 0);
            digests.assign((size_t)n * 32, 0);
            for (int b = 0; b < n; ++b) {
                if (src->fill(src->user, b, scratch.data(), ext) != 0) {
                    set_error("cache_publish: fill failed for block " + std::to_string(b));
                    return LWO_EINVAL;
                }
                Sha256 h;
                h.update(scratch.data(), ext);
                h.final(&digests[(size_t)b * 32]);
            }
        }
        const std::string meta = canonical_meta(d, L);
        uint8_t cd[32];
        content_digest(meta, digests, cd);
        const std::string key = hex(cd, 32);
        std::memcpy(key_out, key.c_str(), 65);

        // Ownership: an exclusive flock on <dir>/<key>.lock, polled up to wait_ms.
        const std::string root = dir, entry = root + "/" + key, lockp = entry + ".lock";
        ::mkdir(root.c_str(), 0755);
        const int lfd = ::open(lockp.c_str(), O_RDWR | O_CREAT | O_CLOEXEC, 0644);
        if (lfd < 0) { set_error("cache_publish: cannot open " + lockp + ": " + std::strerror(errno)); return LWO_EIO; }
        const auto t0 = std::chrono::steady_clock::now();
        while (::flock(lfd, LOCK_EX | LOCK_NB) != 0) {
            if (errno != EWOULDBLOCK && errno != EINTR) {
                ::close(lfd);
                set_error(std::string("cache_publish: flock: ") + std::strerror(errno));
                return LWO_EIO;
            }
            if (std::chrono::steady_clock::now() - t0 >= std::chrono::milliseconds(wait_ms)) {
                ::close(lfd);
                set_error("cache_publish: another writer holds " + lockp);
                return LWO_ETIMEOUT;
            }
            std::this_thread::sleep_for(std::chrono::milliseconds(5));
        }
        auto unlock = [&] { ::flock(lfd, LOCK_UN); ::close(lfd); };

        if (exists(entry + "/manifest.json")) {   // published before: join it
            unlock();
            return LWO_OK;
        }
        // Stale temporaries of this key belong to writers that died holding the lock.
        if (DIR* dd = ::opendir(root.c_str())) {
            const std::string pre = ".tmp-" + key + "-";
            std::vector<std::string> stale;
            while (struct dirent* e = ::readdir(dd))
                if (std::strncmp(e->d_name, pre.c_str(), pre.size()) == 0) stale.push_back(root + "/" + e->d_name);
            ::closedir(dd);
            for (const std::string& p : stale) remove_tree(p);
        }
        std::mt19937_64 rng((uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() ^ (uint64_t)::getpid());
        const std::string tmp = root + "/.tmp-" + key + "-" + std::to_string(::getpid()) + "-" + std::to_string(rng() % 1000000);
        if (::mkdir(tmp.c_str(), 0755) != 0) {
            unlock();
            set_error("cache_publish: cannot create " + tmp + ": " + std::strerror(errno));
            return LWO_EIO;
        }
        auto fail = [&](const std::string& msg) {
            remove_tree(tmp);
            unlock();
            set_error("cache_publish: " + msg);
            return LWO_EIO;
        };
        // Pass 2: blocks.bin (extent, zero padding to the stride).
        {
            const int fd = ::open((tmp + "/blocks.bin").c_str(), O_WRONLY | O_CREAT | O_TRUNC | O_CLOEXEC, 0644);
            if (fd < 0) return fail("cannot create blocks.bin");
            std::vector<uint8_t> pad(stride - ext, 0);
            for (int b = 0; b < n; ++b) {
                const void* p = src->extents ? src->extents[b] : nullptr;
                if (!p) {
                    if (src->fill(src->user, b, scratch.data(), ext) != 0) { ::close(fd); return fail("fill failed on the second pass"); }
                    p = scratch.data();
                }
                if (!write_all(fd, p, ext) || (pad.size() && !write_all(fd, pad.data(), pad.size()))) {
                    ::close(fd);
                    return fail("write of blocks.bin failed");
                }
            }
            const bool ok = ::fsync(fd) == 0;
            ::close(fd);
            if (!ok) return fail("fsync of blocks.bin failed");
        }
        {
            const std::string j = manifest_json(d, L, meta, stride, digests, key);
            const int fd = ::open((tmp + "/manifest.json").c_str(), O_WRONLY | O_CREAT | O_TRUNC | O_CLOEXEC, 0644);
            if (fd < 0) return fail("cannot create manifest.json");
            const bool ok = write_all(fd, j.data(), j.size()) && ::fsync(fd) == 0;
            ::close(fd);
            if (!ok) return fail("write of manifest.json failed");
        }
        if (!fsync_path(tmp, O_RDONLY | O_DIRECTORY)) return fail("fsync of the temporary directory failed");
        if (::rename(tmp.c_str(), entry.c_str()) != 0) return fail(std::string("rename failed: ") + std::strerror(errno));
        (void)fsync_path(root, O_RDONLY | O_DIRECTORY);
        unlock();
        *created = 1;
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_cache_publish");
    } catch (const std::exception& e) {
        return fail_exception("lwo_cache_publish", e.what());
    } catch (...) {
        return fail_exception("lwo_cache_publish", "unknown exception");
    }
}

extern "C" lwo_status lwo_cache_open(const char* dir, const char* key, const lwo_model_desc* desc, int32_t verify,
                                     lwo_cache** out) {
    try {
        clear_error();
        if (!dir || !key || !desc || !out) { set_error("cache_open: NULL argument"); return LWO_EINVAL; }
        *out = nullptr;
        LWO_TRY(validate_desc(desc));
        const Layout L = make_layout(*desc);
        const uint64_t ext = L.extent_bytes, stride = (ext + kPage - 1) / kPage * kPage;
        const int n = desc->n_blocks;
        const std::string entry = std::string(dir) + "/" + key;
        std::string j;
        if (!read_file(entry + "/manifest.json", j)) { set_error("cache_open: no manifest in " + entry); return LWO_EIO; }
        std::string fmt, meta, cdhex;
        uint64_t m_ext = 0, m_stride = 0, m_n = 0, m_file = 0;
        std::vector<uint8_t> digests;
        if (!json_string(j, "format", fmt) || fmt != kFormat || !json_string(j, "meta", meta) ||
            !json_string(j, "content_digest", cdhex) || !json_u64(j, "extent_bytes", m_ext) ||
            !json_u64(j, "stride", m_stride) || !json_u64(j, "n_blocks", m_n) || !json_u64(j, "file_bytes", m_file) ||
            !json_digest_list(j, "block_sha256", (int)m_n, digests)) {
            set_error("cache_open: malformed manifest in " + entry);
            return LWO_EIO;
        }
        if (meta != canonical_meta(*desc, L) || m_ext != ext || m_stride != stride || m_n != (uint64_t)n ||
            m_file != stride * (uint64_t)n) {
            set_error("cache_open: the entry was published for a different block layout");
            return LWO_EINVAL;
        }
        uint8_t cd[32];
        content_digest(meta, digests, cd);
        if (hex(cd, 32) != cdhex || cdhex != key) {
            set_error("cache_open: content digest does not match the key");
            return LWO_ECHECKSUM;
        }
        lwo_cache* c = new (std::nothrow) lwo_cache();
        if (!c) { set_error("out of host memory"); return LWO_ENOMEM; }
        c->fd = ::open((entry + "/blocks.bin").c_str(), O_RDONLY | O_CLOEXEC);
        struct stat st;
        if (c->fd < 0 || ::fstat(c->fd, &st) != 0 || (uint64_t)st.st_size != m_file) {
            lwo_cache_close(c);
            set_error("cache_open: blocks.bin is missing or has the wrong size");
            return LWO_EIO;
        }
        c->map_bytes = m_file;
        c->base = ::mmap(nullptr, m_file, PROT_READ, MAP_SHARED, c->fd, 0);
        if (c->base == MAP_FAILED) {
            c->base = nullptr;
            lwo_cache_close(c);
            set_error(std::string("cache_open: mmap failed: ") + std::strerror(errno));
            return LWO_EIO;
        }
        c->extents.resize(n);
        std::vector<const uint8_t*> ptr(n);
        for (int b = 0; b < n; ++b) ptr[b] = (const uint8_t*)c->base + stride * (uint64_t)b, c->extents[b] = ptr[b];
        if (verify) {
            std::vector<uint8_t> got;
            block_digests(ptr, ext, got);
            for (int b = 0; b < n; ++b)
                if (std::memcmp(&got[(size_t)b * 32], &digests[(size_t)b * 32], 32) != 0) {
                    lwo_cache_close(c);
                    set_error("cache_open: block " + std::to_string(b) + " does not match its manifest digest");
                    return LWO_ECHECKSUM;
                }
        }
        *out = c;
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_cache_open");
    } catch (const std::exception& e) {
        return fail_exception("lwo_cache_open", e.what());
    } catch (...) {
        return fail_exception("lwo_cache_open", "unknown exception");
    }
}

extern "C" lwo_status lwo_cache_extents(const lwo_cache* c, const void** out, int32_t cap, int32_t* n) {
    try {
        clear_error();
        if (!c) { set_error("cache_extents: NULL cache"); return LWO_EINVAL; }
        if (n) *n = (int32_t)c->extents.size();
        if (!out && cap == 0) return LWO_OK;
        if (!out || cap < (int32_t)c->extents.size()) { set_error("cache_extents: capacity too small"); return LWO_EINVAL; }
        for (size_t b = 0; b < c->extents.size(); ++b) out[b] = c->extents[b];
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_cache_extents");
    } catch (const std::exception& e) {
        return fail_exception("lwo_cache_extents", e.what());
    } catch (...) {
        return fail_exception("lwo_cache_extents", "unknown exception");
    }
}

extern "C" lwo_status lwo_cache_close(lwo_cache* c) {
    try {
        clear_error();
        if (!c) return LWO_OK;
        if (c->base) ::munmap(c->base, c->map_bytes);
        if (c->fd >= 0) ::close(c->fd);
        delete c;
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_cache_close");
    } catch (const std::exception& e) {
        return fail_exception("lwo_cache_close", e.what());
    } catch (...) {
        return fail_exception("lwo_cache_close", "unknown exception");
    }
}
