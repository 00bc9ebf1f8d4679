// Memory-mappable weight container for packed models.
//
// The pages' runtime loads its weights from a custom mmap-able binary with a
// fixed 256-byte header that opens with an 8-byte magic string, checked
// before anything else so that a wrong file is refused instead of being
// uploaded ("Building a Custom LLM Inference Runtime for Qwen2.5-Coder-7B on
// NVIDIA H100 Hopper Architecture", section ".nanoqwen File Format and Safety
// Protocols"; "The Architecture of Modern Inference…", section "Data Integrity
// and Serialization").  The same shape is kept here, holding the gfx950
// packed layout instead of the pages' Hopper one, hence its own magic:
//
//   header (256 bytes, little-endian):
//     0   magic "W4GFX950"          8   u32 version (1)   12  u32 header bytes (256)
//     16  u32 tensor count          20  u32 table entry bytes (96)
//     24  u64 table offset (256)    32  u64 file bytes
//     40  u64 FNV-1a 64 of the table
//     48  w4_model_config (48 bytes, max_pages unused)
//     96..255 zero
//   table: one 96-byte entry per tensor:
//     0 name (48 bytes, NUL-terminated)   48 u32 kind   52 u32 row order
//     56 i64 rows   64 i64 cols   72 u64 offset   80 u64 bytes   88 u64 0
//   data: each tensor at a 4096-byte aligned offset, in table order.
//
// Opening validates, in order: size, magic, version, header and entry sizes,
// the table's bounds and checksum, then every entry (NUL-terminated name,
// known kind, byte count equal to what the kind and shape imply, alignment,
// bounds, no overlap).  The first failure is returned as W4_EFORMAT with a
// message; nothing is mapped after a failure.
#include <fcntl.h>
#include <stdio.h>
#include <string.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <vector>

#include "w4_common.hpp"

namespace w4 {
w4_status fail(w4_status code, const char *fmt, ...);
void clear_error();
}  // namespace w4

using namespace w4;

namespace {

constexpr char kMagic[8] = {'W', '4', 'G', 'F', 'X', '9', '5', '0'};
constexpr uint32_t kVersion = 1;
constexpr uint32_t kHeaderBytes = 256;
constexpr uint32_t kEntryBytes = 96;
constexpr uint64_t kAlign = 4096;

#pragma pack(push, 1)
struct Header {
    char magic[8];
    uint32_t version, header_bytes, n_tensors, entry_bytes;
    uint64_t table_offset, file_bytes, table_hash;
    w4_model_config cfg;
    uint8_t pad[kHeaderBytes - 96];
};
struct Entry {
    char name[48];
    uint32_t kind, order;
    int64_t rows, cols;
    uint64_t offset, bytes, reserved;
};
#pragma pack(pop)
static_assert(sizeof(w4_model_config) == 48, "w4_model_config layout");
static_assert(sizeof(Header) == kHeaderBytes, "header size");
static_assert(sizeof(Entry) == kEntryBytes, "entry size");

uint64_t fnv1a64(const void *p, size_t n) {
    const unsigned char *b = static_cast<const unsigned char *>(p);
    uint64_t h = 1469598103934665603ull;
    for (size_t i = 0; i < n; ++i) {
        h ^= b[i];
        h *= 1099511628211ull;
    }
    return h;
}

// Bytes a tensor of this kind and shape must hold (0: invalid).
size_t expected_bytes(uint32_t kind, int64_t rows, int64_t cols) {
    if (rows < 1 || cols < 1 || rows > (int64_t(1) << 31) || cols > (int64_t(1) << 30)) return 0;
    switch (kind) {
        case W4C_INT4_CODES: return w4_packed_qbytes(rows, cols);
        case W4C_INT4_SCALES: return w4_packed_sbytes(rows, cols);
        case W4C_F16: return static_cast<size_t>(rows) * static_cast<size_t>(cols) * 2;
        case W4C_F16_ROWS: return w4_packed_f16_bytes(rows, cols);
        default: return 0;
    }
}

uint64_t align_up(uint64_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

}  // namespace

struct w4c_file {
    void *map = nullptr;
    size_t size = 0;
    const Header *hdr = nullptr;
    const Entry *table = nullptr;
};

extern "C" {

w4_status w4c_write(const char *path, const w4_model_config *cfg, int32_t n, const w4c_tensor *tensors) {
    clear_error();
    if (!path || !cfg || !tensors || n < 1) return fail(W4_EINVAL, "w4c_write: bad arguments");
    std::vector<Entry> table(static_cast<size_t>(n));
    uint64_t off = align_up(kHeaderBytes + static_cast<uint64_t>(n) * kEntryBytes);
    for (int32_t i = 0; i < n; ++i) {
        const w4c_tensor &t = tensors[i];
        Entry &e = table[i];
        memset(&e, 0, sizeof e);
        if (!t.name || strlen(t.name) >= sizeof e.name) return fail(W4_EINVAL, "tensor %d: name missing or too long", i);
        const size_t want = expected_bytes(static_cast<uint32_t>(t.kind), t.rows, t.cols);
        if (want == 0 || t.bytes != want || !t.data)
            return fail(W4_EINVAL, "tensor '%s': %zu bytes given, kind %d of %lld x %lld needs %zu", t.name, t.bytes,
                        t.kind, (long long)t.rows, (long long)t.cols, want);
        memcpy(e.name, t.name, strlen(t.name));
        e.kind = static_cast<uint32_t>(t.kind);
        e.order = static_cast<uint32_t>(t.row_order);
        e.rows = t.rows;
        e.cols = t.cols;
        e.offset = off;
        e.bytes = t.bytes;
        off = align_up(off + t.bytes);
    }
    Header h;
    memset(&h, 0, sizeof h);
    memcpy(h.magic, kMagic, 8);
    h.version = kVersion;
    h.header_bytes = kHeaderBytes;
    h.n_tensors = static_cast<uint32_t>(n);
    h.entry_bytes = kEntryBytes;
    h.table_offset = kHeaderBytes;
    h.file_bytes = off;
    h.table_hash = fnv1a64(table.data(), table.size() * kEntryBytes);
    h.cfg = *cfg;
    FILE *f = fopen(path, "wb");
    if (!f) return fail(W4_EINVAL, "cannot create %s", path);
    bool ok = fwrite(&h, sizeof h, 1, f) == 1 && fwrite(table.data(), kEntryBytes, table.size(), f) == table.size();
    static const char zeros[kAlign] = {};
    uint64_t pos = kHeaderBytes + static_cast<uint64_t>(n) * kEntryBytes;
    for (int32_t i = 0; ok && i < n; ++i) {
        while (ok && pos < table[i].offset) {
            const size_t z = static_cast<size_t>(std::min<uint64_t>(table[i].offset - pos, kAlign));
            ok = fwrite(zeros, 1, z, f) == z;
            pos += z;
        }
        ok = ok && fwrite(tensors[i].data, 1, tensors[i].bytes, f) == tensors[i].bytes;
        pos += tensors[i].bytes;
    }
    while (ok && pos < off) {
        const size_t z = static_cast<size_t>(std::min<uint64_t>(off - pos, kAlign));
        ok = fwrite(zeros, 1, z, f) == z;
        pos += z;
    }
    ok = (fclose(f) == 0) && ok;
    return ok ? W4_OK : fail(W4_EINVAL, "write to %s failed", path);
}

w4_status w4c_open(const char *path, w4c_file **out) {
    clear_error();
    if (!path || !out) return fail(W4_EINVAL, "w4c_open: bad arguments");
    *out = nullptr;
    const int fd = open(path, O_RDONLY);
    if (fd < 0) return fail(W4_EINVAL, "cannot open %s", path);
    struct stat st;
    if (fstat(fd, &st) != 0) {
        close(fd);
        return fail(W4_EINVAL, "cannot stat %s", path);
    }
    const size_t size = static_cast<size_t>(st.st_size);
    // the magic is read and checked before the file is mapped
    char magic[8] = {};
    if (size < kHeaderBytes || pread(fd, magic, 8, 0) != 8 || memcmp(magic, kMagic, 8) != 0) {
        close(fd);
        return fail(W4_EFORMAT, "%s: not a weight container (bad magic or shorter than its header)", path);
    }
    void *map = mmap(nullptr, size, PROT_READ, MAP_PRIVATE, fd, 0);
    close(fd);
    if (map == MAP_FAILED) return fail(W4_EINVAL, "cannot map %s", path);
    auto refuse = [&](const char *why) {
        munmap(map, size);
        return fail(W4_EFORMAT, "%s: %s", path, why);
    };
    const Header *h = static_cast<const Header *>(map);
    if (h->version != kVersion) return refuse("unsupported version");
    if (h->header_bytes != kHeaderBytes || h->entry_bytes != kEntryBytes) return refuse("unexpected header or entry size");
    if (h->file_bytes != size) return refuse("file size differs from the header (truncated or padded)");
    if (h->n_tensors == 0 || h->table_offset != kHeaderBytes ||
        h->table_offset + static_cast<uint64_t>(h->n_tensors) * kEntryBytes > size)
        return refuse("tensor table out of bounds");
    const Entry *table = reinterpret_cast<const Entry *>(static_cast<const char *>(map) + h->table_offset);
    if (fnv1a64(table, static_cast<size_t>(h->n_tensors) * kEntryBytes) != h->table_hash)
        return refuse("tensor table checksum mismatch");
    uint64_t end = h->table_offset + static_cast<uint64_t>(h->n_tensors) * kEntryBytes;
    for (uint32_t i = 0; i < h->n_tensors; ++i) {
        const Entry &e = table[i];
        if (memchr(e.name, 0, sizeof e.name) == nullptr || e.name[0] == 0) return refuse("bad tensor name");
        const size_t want = expected_bytes(e.kind, e.rows, e.cols);
        if (want == 0 || e.bytes != want) return refuse("tensor size does not match its kind and shape");
        // (written so that no sum can wrap past 2^64)
        if (e.offset % kAlign || e.offset < end || e.offset > size || e.bytes > size - e.offset)
            return refuse("tensor offset out of order or bounds");
        end = e.offset + e.bytes;
    }
    w4c_file *f = new w4c_file;
    f->map = map;
    f->size = size;
    f->hdr = h;
    f->table = table;
    *out = f;
    return W4_OK;
}

int32_t w4c_count(const w4c_file *f) { return f ? static_cast<int32_t>(f->hdr->n_tensors) : 0; }

w4_status w4c_config(const w4c_file *f, w4_model_config *cfg) {
    clear_error();
    if (!f || !cfg) return fail(W4_EINVAL, "w4c_config: bad arguments");
    *cfg = f->hdr->cfg;
    return W4_OK;
}

w4_status w4c_tensor_at(const w4c_file *f, int32_t i, w4c_tensor *t) {
    clear_error();
    if (!f || !t || i < 0 || i >= static_cast<int32_t>(f->hdr->n_tensors)) return fail(W4_EINVAL, "w4c_tensor_at: bad index");
    const Entry &e = f->table[i];
    t->name = e.name;
    t->kind = static_cast<int32_t>(e.kind);
    t->row_order = static_cast<int32_t>(e.order);
    t->rows = e.rows;
    t->cols = e.cols;
    t->data = static_cast<const char *>(f->map) + e.offset;
    t->bytes = static_cast<size_t>(e.bytes);
    return W4_OK;
}

w4_status w4c_find(const w4c_file *f, const char *name, w4c_tensor *t) {
    clear_error();
    if (!f || !name || !t) return fail(W4_EINVAL, "w4c_find: bad arguments");
    for (uint32_t i = 0; i < f->hdr->n_tensors; ++i)
        if (strncmp(f->table[i].name, name, sizeof f->table[i].name) == 0) return w4c_tensor_at(f, static_cast<int32_t>(i), t);
    return fail(W4_EINVAL, "no tensor named '%s'", name);
}

void w4c_close(w4c_file *f) {
    if (!f) return;
    munmap(f->map, f->size);
    delete f;
}

}  // extern "C"
